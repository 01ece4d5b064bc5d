// Instantiation unit of the column chain (see chain.h): variant static.
#include "chain.h"

namespace gptq {

gptq_status launch_chain_static(const ChainArgs& a, hipStream_t st) {
  return chain::launch_fs<chain::kFsStatic>(a, st);
}

}  // namespace gptq
