// pa_append.hip — writing the T new tokens of each sequence into their paged
// cache slots, the step just before the verify attention reads them.  Token
// b_s + i of sequence s goes to position L_s + i: block
// block_tables[s][(L_s + i) / block_size], slot (L_s + i) % block_size, in the
// tiled page layout of the attention kernels.  For a u8 cache each (token,
// KV head) vector is quantised on the way in: the cache holds u8 KV with f16
// compute (OpenVINO issue #38153 "[GPU] PagedAttention with 2-4 query tokens
// per sequence (speculative decoding verify) is ~8x slower than single-token
// decode", section "Step-by-step reproduction"), per token per KV head,
// asymmetric, f16 scale and zero point.  The steps are IEEE fp32 operations
// in a fixed order, so codes are reproducible bit for bit:
//   s = f16(range / 255), z = f16(-min / s), code = clamp(rne(x / s + z), 0, 255)
// (a constant row, or one whose scale rounds to 0, takes s = 1, z = f16(-min)).
#include "pa_kernels_impl.h"

namespace pav {

namespace {

// Offsets of element (slot, d) inside one (block, KV head) page of bs slots:
// the orders the segment kernel's loads assume (sub-tiles of 16 slots; pages
// of fewer slots: K [slot][d], V [d][slot]).
__device__ __forceinline__ int k_off(int slot, int d, int D, bool u8, int bs) {
  if (bs < 16) return slot * D + d;
  const int st = slot / 16, m = slot % 16;
  if (u8) return (((st * (D / 64) + d / 64) * 4 + (d % 64) / 16) * 16 + m) * 16 + d % 16;
  return (((st * (D / 32) + d / 32) * 4 + (d % 32) / 8) * 16 + m) * 8 + d % 8;
}
__device__ __forceinline__ int v_off(int slot, int d, int D, bool u8, int bs) {
  if (bs < 16) return d * bs + slot;
  const int st = slot / 16, qq = (slot % 16) / 4;
  if (u8) return ((((st * (D / 64) + d / 64) * 4 + qq) * 16 + d % 16) * 4 + (d % 64) / 16) * 4 + slot % 4;
  return ((((st * (D / 32) + d / 32) * 4 + qq) * 16 + d % 16) * 2 + (d % 32) / 16) * 4 + slot % 4;
}

template <int QT>
__device__ __forceinline__ float in_value(const uint16_t* p) {
  const uint16_t b = *p;
  if constexpr (QT == kF16) return (float)__builtin_bit_cast(_Float16, b);
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ float wave_min(float v) { return wave_reduce(v, fmin_op); }

}  // namespace

// One wavefront per (token, KV head, K or V).  Lane l handles d = l + 64*e.
template <int QT, int KV, int D>
__global__ __launch_bounds__(kWave) void pa_append(AppendArgs a) {
  constexpr bool U8 = KV == kU8;
  constexpr int E = D / kWave > 0 ? D / kWave : 1;      // elements per lane
  const int lane = threadIdx.x;
  const int n = blockIdx.x, g = blockIdx.y, kv = blockIdx.z;

  // One wavefront checks subsequence_begins as a whole (starts at 0, never
  // decreases, ends at num_tokens) and sets the status if it is broken; the
  // others take it as sorted.
  if (n == 0 && g == 0 && kv == 0) {
    bool bad = false;
    for (int k = lane; k < a.num_seqs; k += kWave) bad |= a.sb[k] > a.sb[k + 1];
    if (lane == 0) bad |= a.sb[0] != 0 || a.sb[a.num_seqs] != a.num_tokens;
    if (__any(bad) && lane == 0) atomicExch(a.status, kDeviceContract);
  }
  // The token's sequence: the last s with sb[s] <= n, narrowed 64 entries
  // at a time (one load per lane and round: two rounds up to 4096
  // sequences).  Whatever the array holds, a token is written only for an s
  // with sb[s] <= n < sb[s + 1] whose own checks below pass: a position of
  // that sequence's new tokens, inside its block table.
  int lo = 0, cnt = a.num_seqs;                               // candidates sb[lo .. lo + cnt)
  int s = -1;
  while (true) {
    const int stride = cnt > kWave ? (cnt + kWave - 1) / kWave : 1;
    const int k = lo + lane * stride;
    const bool le = lane * stride < cnt && a.sb[k] <= n;
    const unsigned long long m = __ballot(le);
    if (!m) break;                                            // n below every candidate
    const int l = 63 - __builtin_clzll(m);
    if (stride == 1) {
      s = lo + l;
      break;
    }
    lo += l * stride;
    cnt = min(stride, cnt - l * stride);
  }
  bool ok = s >= 0;
  int blk = 0, slot = 0;
  if (ok) {
    const int b0 = a.sb[s], T = a.sb[s + 1] - b0, L = a.past_lens[s];
    const int pos = L + (n - b0);
    ok = n < b0 + T && T >= 1 && T <= a.max_q && L >= 0 && (int64_t)pos < (int64_t)a.mbps * a.bs;
    if (ok) {
      blk = a.bt[(size_t)s * a.mbps + pos / a.bs];
      slot = pos % a.bs;
      ok = blk >= 0 && blk < a.num_blocks;
    }
  }
  if (!ok) {
    if (lane == 0) atomicExch(a.status, kDeviceContract);
    return;
  }

  const uint16_t* src = reinterpret_cast<const uint16_t*>(kv ? a.v_new : a.k_new) +
                        ((size_t)n * a.Hkv + g) * D;
  const size_t page = ((size_t)blk * a.Hkv + g) * a.bs * D;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = lane + e * kWave;
    x[e] = d < D ? in_value<QT>(src + d) : 0.f;
  }
  if constexpr (!U8) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(kv ? a.v_cache : a.k_cache) + page;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = lane + e * kWave;
      if (d < D) dst[a.page_layout == kPagesRowMajor ? slot * D + d
                    : kv ? v_off(slot, d, D, false, a.bs) : k_off(slot, d, D, false, a.bs)] = src[d];
    }
  } else {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) {
      mn = fminf(mn, x[e]);
      mx = fmaxf(mx, x[e]);
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    const _Float16 s_try = (_Float16)__fdiv_rn(__fsub_rn(mx, mn), 255.0f);
    _Float16 sh = (_Float16)1.0f, zh;
    if (mx != mn && s_try != (_Float16)0.0f) {
      sh = s_try;
      zh = (_Float16)__fdiv_rn(-mn, (float)sh);
    } else {
      zh = (_Float16)(-mn);
    }
    const float sf = (float)sh, zf = (float)zh;
    uint8_t* dst = reinterpret_cast<uint8_t*>(kv ? a.v_cache : a.k_cache) + page;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = lane + e * kWave;
      const float r = fminf(fmaxf(rintf(__fadd_rn(__fdiv_rn(x[e], sf), zf)), 0.f), 255.f);
      if (d < D) dst[a.page_layout == kPagesRowMajor ? slot * D + d
                    : kv ? v_off(slot, d, D, true, a.bs) : k_off(slot, d, D, true, a.bs)] = (uint8_t)r;
    }
    if (lane == 0) {
      uint16_t* sz = reinterpret_cast<uint16_t*>(kv ? a.vsz : a.ksz) +
                     (((size_t)blk * a.Hkv + g) * a.bs + slot) * 2;
      sz[0] = __builtin_bit_cast(uint16_t, sh);
      sz[1] = __builtin_bit_cast(uint16_t, zh);
    }
  }
}

template <int QT, int KV>
static hipError_t launch_append_d(const AppendArgs& a, int D, hipStream_t st) {
  const dim3 grid(a.num_tokens, a.Hkv, 2);
  switch (D) {
    case 64: return launch_kernel(reinterpret_cast<const void*>(pa_append<QT, KV, 64>), grid, dim3(kWave), st, a);
    case 128: return launch_kernel(reinterpret_cast<const void*>(pa_append<QT, KV, 128>), grid, dim3(kWave), st, a);
    case 256: return launch_kernel(reinterpret_cast<const void*>(pa_append<QT, KV, 256>), grid, dim3(kWave), st, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_append(const AppendArgs& a, int q_dtype, int kv_dtype, int D, hipStream_t st) {
  if (kv_dtype == kU8)
    return q_dtype == kF16 ? launch_append_d<kF16, kU8>(a, D, st) : launch_append_d<kBF16, kU8>(a, D, st);
  return q_dtype == kF16 ? launch_append_d<kF16, kF16>(a, D, st) : launch_append_d<kBF16, kBF16>(a, D, st);
}

}  // namespace pav
