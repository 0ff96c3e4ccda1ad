// Label range check of the forward pass.
//
// Row u of sample b's lattice emits label y[b, u+1] for u < U_b ("Neural
// transducer training ...", section "Transducer training": the label
// sequence with the blank prepended). Every kernel that indexes the output
// layer by a label reads the copy this kernel writes into `saved`, so a label
// outside [0, V) can never address memory outside W^O, b^O or a score row:
// such a label is replaced by the blank id in the copy and counted. Columns
// past U_b (never read from the caller's array) and column 0 are written as
// the blank id.
#include "common.hpp"
#include "kernels.hpp"

namespace rnnt {

// One workgroup: B * (U+1) is at most a few hundred thousand entries.
__global__ void __launch_bounds__(1024) labels_check_kernel(const int32_t* __restrict__ labels,
                                                            const int32_t* __restrict__ U_len, int B, int U1, int V,
                                                            int blank, int32_t* __restrict__ out,
                                                            int32_t* __restrict__ status) {
  __shared__ int s_cnt[16], s_first[16];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)B * U1;
  int cnt = 0, first = 0x7fffffff;
  for (int64_t i = tid; i < n; i += 1024) {
    const int b = (int)(i / U1), c = (int)(i - (int64_t)b * U1);
    int lab = blank;
    if (c >= 1 && c <= U_len[b]) {
      const int y = labels[i];
      const bool bad = y < 0 || y >= V;
      cnt += bad ? 1 : 0;
      if (bad && i < first) first = (int)i;
      lab = bad ? blank : y;
    }
    out[i] = lab;
  }
  // wave sums / minima, then across the 16 waves
  for (int o = 32; o > 0; o >>= 1) {
    cnt += __shfl_xor(cnt, o);
    first = min(first, __shfl_xor(first, o));
  }
  if ((tid & 63) == 0) {
    s_cnt[tid >> 6] = cnt;
    s_first[tid >> 6] = first;
  }
  __syncthreads();
  if (tid == 0) {
    int c = 0, f = 0x7fffffff;
    for (int w = 0; w < 16; ++w) {
      c += s_cnt[w];
      f = min(f, s_first[w]);
    }
    status[0] = c;
    status[1] = c ? f : -1;
  }
}

hipError_t launch_labels_check(const int32_t* labels, const int32_t* U_len, int B, int U1, int V, int blank,
                               int32_t* out, int32_t* status, hipStream_t st) {
  if ((int64_t)B * U1 >= 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(labels_check_kernel, dim3(1), dim3(1024), 0, st, labels, U_len, B, U1, V, blank, out, status);
  return hipGetLastError();
}

}  // namespace rnnt
