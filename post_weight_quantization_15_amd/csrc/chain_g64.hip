// Instantiation unit of the column chain (see chain.h): variant g64.
#include "chain.h"

namespace gptq {

gptq_status launch_chain_g64(const ChainArgs& a, hipStream_t st) {
  return chain::launch_fs<64>(a, st);
}

}  // namespace gptq
