// Page-sharded ownership closed form ("HiCache across parallel modes and distributed
// serving", §1.1): logical page q = floor(x/p), owner r = q mod N, owner-local row
// floor(q/N)*p + (x mod p).  Pure arithmetic, one thread per slot.
#include "common.h"

namespace dsa {

__global__ void __launch_bounds__(256) page_translate_kernel(const int64_t* __restrict__ x, int64_t n,
                                                             int64_t p, int64_t N, int32_t* __restrict__ rank,
                                                             int64_t* __restrict__ local_row, int32_t* err) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t xi = x[i];
    if (xi < 0) {
      rank[i] = -1;
      local_row[i] = -1;
      count_error(err);
      continue;
    }
    const int64_t q = xi / p;
    rank[i] = (int32_t)(q % N);
    local_row[i] = (q / N) * p + (xi - q * p);
  }
}

}  // namespace dsa

extern "C" dsa_status_t dsa_page_translate(const int64_t* x, int64_t n, int page_size, int n_ranks,
                                           int32_t* rank, int64_t* local_row, int32_t* err_count,
                                           hipStream_t stream) {
  DSA_CHECK_ARG(n >= 0, "dsa_page_translate: n < 0");
  DSA_CHECK_ARG(page_size > 0 && n_ranks > 0, "dsa_page_translate: page_size and n_ranks must be > 0");
  if (n == 0) return DSA_OK;
  DSA_CHECK_ARG(x && rank && local_row, "dsa_page_translate: null pointer");
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  DSA_LAUNCH(dsa::page_translate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, n,
                     (int64_t)page_size, (int64_t)n_ranks, rank, local_row, err_count);
  return dsa::launch_status("dsa_page_translate");
}
