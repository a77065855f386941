// Device-side check of the per-sequence inputs of the paged decode (gfx950).
//
// The decode reads the sequence lengths and the block table from device
// memory and trusts them: a length below the query count, or a page id
// outside the cache, is not detectable on the host.  This kernel counts such
// violations for a caller that wants to know (debug runs, tests).  The
// conditions are those the decode's contract states for its inputs: the
// record cache is paged (pages of block_size records, a table of physical
// page ids per sequence), and sequence b holds seq_lens[b] records of which
// the last S_q are the queries' own positions.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

// One work-group walks every (sequence, entry) pair, entry -1 standing for
// the length itself; the count is reduced through LDS and written by thread 0.
__global__ void __launch_bounds__(1024) validate_kernel(ValidateParams p) {
  __shared__ int partial[1024 / kWave];
  const int64_t per = (int64_t)p.MB + 1;
  const int64_t total = (int64_t)p.B * per;
  const int64_t cap = (int64_t)p.MB * p.block_size;
  int bad = 0;
  for (int64_t e = threadIdx.x; e < total; e += blockDim.x) {
    const int b = (int)(e / per);
    const int64_t j = e % per - 1;
    const int L = p.seq_lens[b];
    const bool len_ok = L == 0 || (L >= p.S && (int64_t)L <= cap);
    if (j < 0) {
      bad += len_ok ? 0 : 1;
    } else if (len_ok && j < ((int64_t)L + p.block_size - 1) / p.block_size) {
      const int page = p.block_table[(int64_t)b * p.MB + j];
      bad += (page < 0 || (int64_t)page >= p.num_pages) ? 1 : 0;
    }
  }
  int s = bad;
  for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((threadIdx.x & (kWave - 1)) == 0) partial[threadIdx.x / kWave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < (int)(blockDim.x / kWave); ++i) t += partial[i];
    *p.out = t;
  }
}

}  // namespace

hipError_t launch_validate(const ValidateParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
