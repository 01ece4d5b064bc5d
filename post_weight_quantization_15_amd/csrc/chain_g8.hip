// Instantiation unit of the column chain (see chain.h): variant g8.
#include "chain.h"

namespace gptq {

gptq_status launch_chain_g8(const ChainArgs& a, hipStream_t st) {
  return chain::launch_fs<8>(a, st);
}

}  // namespace gptq
