// cache_append.hip — writes the rows of new tokens into the shared caches.
//
// Every extra token of context adds one K row and one V row to the cache
// (CLSA article, opening section), and in the KV-sharing architectures CLSA
// builds on that cache is written once and read by every cross-decoder
// layer (CLSA article, "Comment CLSA fonctionne"); the indexer keys of the
// token go with them. Token t of batch element b lands at cache row
// pos + t; bytes are copied unchanged.
#include "kernels.h"

namespace clsa {
namespace {

constexpr int kAppendThreads = 256;

// grid (B*T rows, n jobs), block kAppendThreads: workgroup (r, j) copies row
// r of job j.
__global__ __launch_bounds__(kAppendThreads) void append_rows(AppendJob j0, AppendJob j1, AppendJob j2, int T,
                                                   int pos, int L_cap) {
  const AppendJob& j = blockIdx.y == 0 ? j0 : (blockIdx.y == 1 ? j1 : j2);
  const size_t r = blockIdx.x;
  const size_t b = r / T, t = r % T;
  const char* src = j.src + r * j.row_bytes;
  char* dst = j.dst + (b * L_cap + pos + t) * j.row_bytes;
  if (j.row_bytes % 16 == 0) {  // 16-byte aligned rows: one uint4 per thread per pass
    for (size_t i = threadIdx.x * 16; i < j.row_bytes; i += kAppendThreads * 16)
      *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
  } else {
    for (size_t i = threadIdx.x; i < j.row_bytes; i += kAppendThreads) dst[i] = src[i];
  }
}

}  // namespace

int launch_cache_append(const AppendJob* jobs, int n_jobs, int B, int T, int pos, int L_cap,
                        hipStream_t stream) {
  const AppendJob none{nullptr, nullptr, 0};
  hipLaunchKernelGGL(append_rows, dim3((unsigned)((size_t)B * T), (unsigned)n_jobs), dim3(kAppendThreads), 0,
                     stream, jobs[0], n_jobs > 1 ? jobs[1] : none, n_jobs > 2 ? jobs[2] : none, T,
                     pos, L_cap);
  return check_launch("append_rows");
}

}  // namespace clsa
