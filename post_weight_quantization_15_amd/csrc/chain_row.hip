// Instantiation unit of the column chain (see chain.h): variant row.
#include "chain.h"

namespace gptq {

gptq_status launch_chain_row(const ChainArgs& a, hipStream_t st) {
  return chain::launch_fs<chain::kFsRow>(a, st);
}

}  // namespace gptq
