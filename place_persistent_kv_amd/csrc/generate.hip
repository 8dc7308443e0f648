// The bookkeeping of one iteration of the generation loop (gfx950).
//
// "Persistent input/output feedback", section "Autoregressive generation":
// the output holds the prompt and every generated token; generation stops
// once every row has emitted EOS; a finished row is padded with
// pad_token_id.  Per row: the token written at this iteration's column is
// the sampled id, or the pad token when the row had already finished; the
// row finishes when the written token is EOS; the written token is also the
// row's next input.  The rows still running are counted so that the host can
// stop the loop.  One workgroup; B is small next to one decode step.  A
// second kernel advances device-held positions and the step counter of a
// captured decode step.

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kGenThreads = 256;

__global__ __launch_bounds__(kGenThreads) void generate_finish_kernel(GenerateArgs a) {
    __shared__ int s_cnt[kGenThreads / 64];
    int cnt = 0;
    for (int b = threadIdx.x; b < a.B; b += kGenThreads) {
        const bool was = a.finished[b] != 0;
        const int64_t tok = was ? a.pad : a.sampled[b];
        const bool now = was || (a.has_eos && tok == a.eos);
        a.finished[b] = now ? 1 : 0;
        a.tokens[int64_t(b) * a.row_stride + a.column] = tok;
        a.next_ids[b] = tok;
        cnt += now ? 0 : 1;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        int total = 0;
        for (int w = 0; w < kGenThreads / 64; ++w) total += s_cnt[w];
        *a.unfinished = total;
    }
}

// Positions or lengths held on the device move on by `delta` and the step
// counter by one, so that a captured decode step can be replayed as is.
__global__ __launch_bounds__(kGenThreads) void advance_kernel(AdvanceArgs a) {
    for (int i = blockIdx.x * kGenThreads + threadIdx.x; i < a.n; i += gridDim.x * kGenThreads)
        a.values[i] += a.delta;
    if (a.step != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *a.step += 1;
}

}  // namespace

hipError_t launch_advance(const AdvanceArgs& a, hipStream_t s) {
    const int blocks = a.n > 0 ? (a.n + kGenThreads - 1) / kGenThreads : 1;
    hipLaunchKernelGGL(advance_kernel, dim3(blocks < 64 ? blocks : 64), dim3(kGenThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_generate_finish(const GenerateArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(generate_finish_kernel, dim3(1), dim3(kGenThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace pkv
