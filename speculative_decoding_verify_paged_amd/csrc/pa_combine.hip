// pa_combine.hip — the segment-combine kernel (log-sum-exp merge of the
// per-token segment partials, cast to the output dtype) and its launcher.
#include "pa_kernels_impl.h"

namespace pav {

// ---------------------------------------------------------------------------
// Combine kernel: one workgroup per (token, q head) (placed by CombineArgs::xcds
// on the XCD that wrote the pair's partials), NT threads with NT sized
// by the host so all S partials are loaded in one batch of K per thread.  Thread t owns d columns
// [c4, c4 + 4) of the segments sub, sub + NSUB, ...; it merges them with the
// same online rescaling as the segment kernel (every load independent of the
// previous iteration's arithmetic, so they all go out at once), then the
// NSUB partial states are merged through LDS in a fixed order.
// ---------------------------------------------------------------------------
template <int D, int OUT, int NT>
__global__ __launch_bounds__(NT) void pa_combine(CombineArgs a) {
  constexpr int LPS = D / 4;                                  // threads per segment row
  constexpr int NSUB = NT / LPS;                              // segment rows in flight
  constexpr int K = 8;                                        // partials per thread per batch
  __shared__ float s_m[NSUB];
  __shared__ float s_den[NSUB];
  __shared__ __attribute__((aligned(16))) f32x4 s_acc[NSUB][LPS];

  int pair = blockIdx.x;                                      // token * Hq + q head
  if (a.xcds > 0) {
    // the pairs of KV heads x, x + xcds, ... in (token, KV head, group) order
    const int X = a.xcds, x = (int)blockIdx.x % X, k = (int)blockIdx.x / X;
    const int G = a.seg.G, HX = a.seg.Hkv / X;
    const int g = k % G, t = k / G;
    pair = (t / HX) * a.Hq + ((t % HX) * X + x) * G + g;
  }
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int sub = tid / LPS;
  const int col = tid % LPS;
  const int n = pair / a.Hq;
  const int S = a.seg.S;

  // subsequence_begins, 64 entries per lane step: its first chunk goes out
  // with the partial loads
  const int nseq = a.seg.num_seqs;
  const int sb_next = lane < nseq ? a.seg.sb[lane + 1] : 0;
  const int sb_this = lane < nseq ? a.seg.sb[lane] : 0;

  // Every segment of a valid sequence wrote its partial (empty ones as
  // (-inf, 0)), so these loads depend on nothing but the grid position.  They
  // are unconditional (clamped index) so they all go out together.
  const float* ml = a.seg.ws_ml + (size_t)pair * S * 2;
  const float* op = a.seg.ws_o + (size_t)pair * S * D + col * 4;
  float m = -INFINITY, den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bool nan_seen = false;
  for (int b = 0; b < S; b += NSUB * K) {
    float mj[K], lj[K];
    f32x4 oj[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int jj = b + sub + k * NSUB;
      const int jc = jj < S ? jj : 0;
      mj[k] = ml[jc * 2];
      lj[k] = ml[jc * 2 + 1];
      oj[k] = *reinterpret_cast<const f32x4*>(op + (size_t)jc * D);
      mj[k] = jj < S ? mj[k] : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      nan_seen |= mj[k] != mj[k];
      const float m_new = fmaxf(m, mj[k]);
      const float base = m_new == -INFINITY ? 0.f : m_new;
      const float sc = __builtin_amdgcn_exp2f(m - base);
      const float f = __builtin_amdgcn_exp2f(mj[k] - base);
      // a segment in which this row saw no key left its O slot unwritten
      const f32x4 o = mj[k] == -INFINITY ? f32x4{0.f, 0.f, 0.f, 0.f} : oj[k];
      den = den * sc + f * lj[k];
      acc = acc * sc + f * o;
      m = m_new;
    }
  }

  // subsequence_begins must start at 0, never decrease and end at
  // num_tokens; then token n belongs to the first s with n < sb[s + 1].  A
  // sequence that breaks the rest of the contract left NaN in its partials.
  bool ok = true;
  int s = -1;
  {
    ok &= !__any(lane < nseq && sb_this > sb_next);
    ok &= __shfl(sb_this, 0, kWave) == 0;
    if (nseq <= kWave) ok &= __shfl(sb_next, nseq - 1, kWave) == a.seg.num_tokens;
    const unsigned long long hit = __ballot(lane < nseq && n < sb_next);
    if (hit) s = __builtin_ctzll(hit);
  }
  for (int b = kWave; b < nseq; b += kWave) {                 // more than 64 sequences
    const int k = b + lane;
    const int nx = k < nseq ? a.seg.sb[k + 1] : 0;
    const int th = k < nseq ? a.seg.sb[k] : 0;
    ok &= !__any(k < nseq && th > nx);
    if (b + kWave >= nseq) ok &= __shfl(nx, nseq - 1 - b, kWave) == a.seg.num_tokens;
    const unsigned long long hit = __ballot(k < nseq && n < nx);
    if (s < 0 && hit) s = b + __builtin_ctzll(hit);
  }
  ok &= s >= 0;
  if (col == 0) {
    s_m[sub] = m;
    s_den[sub] = den;
  }
  s_acc[sub][col] = acc;
  const bool bad = __syncthreads_or(nan_seen || !ok);
  if (bad && tid == 0) atomicExch(a.seg.status, kDeviceContract);
  if (tid >= LPS) return;
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < NSUB; ++k) M = fmaxf(M, s_m[k]);
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float dsum = 0.f;
#pragma unroll
  for (int k = 0; k < NSUB; ++k) {
    const float f = s_m[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[k] - M);
    num += f * s_acc[k][tid];
    dsum += f * s_den[k];
  }
  float res[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) res[k] = bad ? NAN : num[k] / dsum;
  if constexpr (OUT == kF16) {
    _Float16* out = reinterpret_cast<_Float16*>(a.out) + (size_t)pair * D + tid * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = (_Float16)res[k];
  } else {
    __bf16* out = reinterpret_cast<__bf16*>(a.out) + (size_t)pair * D + tid * 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = (__bf16)res[k];
  }
}


template <int D, int NT>
static hipError_t launch_combine_nt(const CombineArgs& a, int out_dtype, dim3 grid, hipStream_t st) {
  const void* fn = out_dtype == kF16 ? reinterpret_cast<const void*>(pa_combine<D, kF16, NT>)
                                     : reinterpret_cast<const void*>(pa_combine<D, kBF16, NT>);
  return launch_kernel(fn, grid, dim3(NT), st, a);
}

template <int D>
static hipError_t launch_combine_d(const CombineArgs& a, int out_dtype, int threads, dim3 grid,
                                   hipStream_t st) {
  switch (threads) {
    case 256: return launch_combine_nt<D, 256>(a, out_dtype, grid, st);
    case 512: return launch_combine_nt<D, 512>(a, out_dtype, grid, st);
    case 1024: return launch_combine_nt<D, 1024>(a, out_dtype, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, int out_dtype, int D, int threads, dim3 grid,
                          hipStream_t st) {
  switch (D) {
    case 64: return launch_combine_d<64>(a, out_dtype, threads, grid, st);
    case 128: return launch_combine_d<128>(a, out_dtype, threads, grid, st);
    case 256: return launch_combine_d<256>(a, out_dtype, threads, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pav
