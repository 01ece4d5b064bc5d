// Instantiation unit of the column chain (see chain.h): variant g128.
#include "chain.h"

namespace gptq {

gptq_status launch_chain_g128(const ChainArgs& a, hipStream_t st) {
  return chain::launch_fs<128>(a, st);
}

}  // namespace gptq
