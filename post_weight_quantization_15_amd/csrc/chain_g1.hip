// Instantiation unit of the column chain (see chain.h): variant g1.
#include "chain.h"

namespace gptq {

gptq_status launch_chain_g1(const ChainArgs& a, hipStream_t st) {
  return chain::launch_fs<1>(a, st);
}

}  // namespace gptq
