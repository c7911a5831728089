// pa_combine.hip — the segment-combine kernel (log-sum-exp merge of the
// per-token segment partials, cast to the output dtype) and its launcher.
#include "pa_kernels_impl.h"

namespace pav {

// ---------------------------------------------------------------------------
// Combine kernel: one wavefront per (token, q head) row and 64-column slice
// of it, each lane owning one output column; the slices of a row are placed
// by CombineArgs::xcds on the XCD that wrote the row's partials.  Every
// segment's (m, l) and the slice's columns of every segment's O go out as
// one batch of independent loads (up to 64 segments per batch); the row max
// and the weighted sum of l are wavefront reductions, and each segment's
// weight reaches all lanes by readlane, so the merge is one dependent round
// trip to memory with no LDS and no barrier.  Slicing the row spreads its
// partials over D / 64 workgroups (and CUs) instead of one.
// ---------------------------------------------------------------------------
constexpr int kCombineBatch = 64;                             // segments per batch: one per lane

template <int D, int OUT>
__global__ __launch_bounds__(kWave) void pa_combine(CombineArgs a) {
  constexpr int CPL = 1;                                      // columns per lane
  constexpr int NSL = D / kWave;                              // slices per row
  int pair, slice;                                            // pair = token * Hq + q head
  if (a.xcds > 0) {
    // the pairs of KV heads x, x + xcds, ... in (token, KV head, group) order,
    // all slices of a pair on the same XCD
    const int X = a.xcds, x = (int)blockIdx.x % X, k = (int)blockIdx.x / X;
    slice = k % NSL;
    const int kk = k / NSL;
    const int G = a.seg.G, HX = a.seg.Hkv / X;
    const int g = kk % G, t = kk / G;
    pair = (t / HX) * a.Hq + ((t % HX) * X + x) * G + g;
  } else {
    pair = (int)blockIdx.x / NSL;
    slice = (int)blockIdx.x % NSL;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int col = slice * kWave + lane;
  const int S = a.seg.S;

  // the segment kernel's verdict on subsequence_begins (one word per
  // wavefront of its workgroup 0): it goes out with the partial loads
  const int sb_bad = lane < a.seg.sb_words ? a.seg.sb_check[lane] : 0;

  // Every segment of a valid sequence wrote its (m, l) (empty ones as
  // (-inf, 0)); a segment in which the row saw no key left its O unwritten,
  // so its O is never read into the sum.  The loads depend on nothing but
  // the grid position and go out together.
  const float* ml = a.seg.ws_ml + (size_t)pair * S * 2;
  const float* op = a.seg.ws_o + (size_t)pair * S * D + col;
  float M = -INFINITY, den = 0.f;
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  bool nan_seen = false;
  // one batch of up to NB segments starting at b (NB: the smallest of 8, 16,
  // 32, 64 that holds the rest, so no more loads than needed go out)
  auto batch = [&](auto nb_tag, int b) {
    constexpr int NB = decltype(nb_tag)::value;
    const int nb = min(NB, S - b);
    const int j = b + (lane < nb ? lane : 0);
    float2 mlj = *reinterpret_cast<const float2*>(ml + (size_t)j * 2);
    float o[NB][CPL];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const size_t jc = (size_t)(b + (k < nb ? k : 0));      // in bounds; unused when k >= nb
      if constexpr (CPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(op + jc * D);
        o[k][0] = v.x;
        o[k][1] = v.y;
      } else {
        o[k][0] = op[jc * D];
      }
    }
    if (lane >= nb) mlj = float2{-INFINITY, 0.f};
    nan_seen |= mlj.x != mlj.x;
    const float m_new = fmaxf(M, wave_max(mlj.x));
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float sc = __builtin_amdgcn_exp2f(M - base);
    // weight of this lane's segment; 0 for an empty one (its O is unwritten)
    const float w = mlj.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mlj.x - base);
    den = den * sc + wave_sum(w * mlj.y);
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] *= sc;
    M = m_new;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
      if (wk != 0.f) {                                        // uniform; skips empty segments
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] += wk * o[k][c];
      }
    }
  };
  for (int b = 0; b < S; b += kCombineBatch) {
    const int rest = S - b;
    if (rest <= 8) batch(std::integral_constant<int, 8>{}, b);
    else if (rest <= 16) batch(std::integral_constant<int, 16>{}, b);
    else if (rest <= 32) batch(std::integral_constant<int, 32>{}, b);
    else batch(std::integral_constant<int, kCombineBatch>{}, b);
  }

  // subsequence_begins must start at 0, never decrease and end at
  // num_tokens; then every token belongs to exactly one sequence.  A
  // sequence that breaks the rest of the contract left NaN in its partials.
  const bool ok = !__any(sb_bad != 0);
  const bool bad = __any(nan_seen) || !ok;
  if (bad && threadIdx.x == 0) atomicExch(a.seg.status, kDeviceContract);
  float res[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) res[c] = bad ? NAN : acc[c] / den;
  if constexpr (OUT == kF16) {
    _Float16* out = reinterpret_cast<_Float16*>(a.out) + (size_t)pair * D + col;
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = (_Float16)res[c];
  } else {
    __bf16* out = reinterpret_cast<__bf16*>(a.out) + (size_t)pair * D + col;
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = (__bf16)res[c];
  }
}

// ---------------------------------------------------------------------------
// Check kernel of a direct call (one segment, output written by the segment
// kernel): when the segment kernel's workgroup 0 found subsequence_begins
// broken, every output row becomes NaN and the status word is set, as the
// combine kernel does; otherwise every wavefront exits after one load.
// ---------------------------------------------------------------------------
template <int OUT>
__global__ __launch_bounds__(kFinishThreads) void pa_finish(CombineArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = lane < a.seg.sb_words ? a.seg.sb_check[lane] : 0;
  if (!__any(w != 0)) return;                                 // uniform
  if (blockIdx.x == 0 && threadIdx.x == 0) atomicExch(a.seg.status, kDeviceContract);
  // element stores: out need only be 2-byte aligned (an error path)
  const uint16_t nan1 = OUT == kF16 ? 0x7E00u : 0x7FC0u;
  const size_t n = (size_t)a.num_tokens * a.Hq * a.head_dim;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = nan1;
}

hipError_t launch_finish(const CombineArgs& a, int out_dtype, int threads, dim3 grid, hipStream_t st) {
  if (threads != kFinishThreads) return hipErrorInvalidValue;
  const void* fn = out_dtype == kF16 ? reinterpret_cast<const void*>(pa_finish<kF16>)
                                     : reinterpret_cast<const void*>(pa_finish<kBF16>);
  return launch_kernel(fn, grid, dim3(kFinishThreads), st, a);
}

template <int D>
static hipError_t launch_combine_d(const CombineArgs& a, int out_dtype, dim3 grid, hipStream_t st) {
  const void* fn = out_dtype == kF16 ? reinterpret_cast<const void*>(pa_combine<D, kF16>)
                                     : reinterpret_cast<const void*>(pa_combine<D, kBF16>);
  return launch_kernel(fn, grid, dim3(kWave), st, a);
}

hipError_t launch_combine(const CombineArgs& a, int out_dtype, int D, int threads, dim3 grid,
                          hipStream_t st) {
  if (threads != kWave || grid.x % (D / kWave) != 0) return hipErrorInvalidValue;
  switch (D) {
    case 64: return launch_combine_d<64>(a, out_dtype, grid, st);
    case 128: return launch_combine_d<128>(a, out_dtype, grid, st);
    case 256: return launch_combine_d<256>(a, out_dtype, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pav
