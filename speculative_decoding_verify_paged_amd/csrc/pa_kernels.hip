// pa_kernels.hip — gfx950 kernels of paged verify attention.
//
// Two kernels per call:
//   1. pa_segment_*: one workgroup per (KV segment j, KV head, sequence).  Its
//      wavefronts stream the segment's K/V page tiles straight from HBM into
//      MFMA operand registers, each tile read once for all G*T stacked query
//      rows of the GQA group, and keep an online softmax.  The workgroup
//      merges its wavefronts in LDS and writes one partial (O, m, l) per query
//      row to the workspace, indexed per token.
//   2. pa_combine: log-sum-exp merge of the segment partials of each
//      (token, q head) row, cast to the output dtype.
//
// Why segments: a verify call at batch 1 has only num_kv_heads independent
// KV streams; a kernel that gives each one workgroup idles almost all of the
// GPU (vLLM article "speculative decoding net loss": the use_3d gate passage,
// 128 workgroups falling to 8; OpenVINO issue #38153, "Performance issue
// description": the unpartitioned MIXED scan).  Splitting the key axis into
// segments reduced in parallel restores the parallelism, and the extra query
// rows ride along in the same MFMA tile (same article, direct kernel sweep:
// one extra row costs a fraction of a percent).
//
// Data path of one wavefront step (32 keys, rows r = g*T + i padded to 16):
//   S^T[key, r] = K[key, :] . Q[r, :]     v_mfma_f32_16x16x32_{f16,bf16}, A = K rows
//                                          read from the page (16 B per lane),
//                                          B = Q rows held in registers
//   online softmax over the step's keys per row (lane-local, 2 cross-lane max)
//   O^T[d, r] += V^T[d, key] . P^T[key, r] A = V^T read from the d-major V page
//                                          (8 keys contiguous, 16 B per lane),
//                                          B = P split into hi + lo f16/bf16 parts
// Every lane owns one stacked row r = lane % 16 in all three products, so the
// softmax state and its rescale never leave the lane.  The cross-lane steps
// are two shuffles for the row max and the workgroup merge at the end.
//
// V pages are stored d-major ([block, head, D, block_size]): the PV
// contraction runs over keys, and the MFMA operand wants 8 consecutive keys
// per lane, which that layout makes one 16-byte load instead of eight 2-byte
// gathers or an LDS transpose.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pav {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ u32x4 ld16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <int KV>
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (KV == kF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// Eight softmax weights as two MFMA operands, hi = rne16(p) and
// lo = rne16(p - hi): PV runs on both, so the weights keep ~16 more bits than
// one 16-bit rounding (bf16 alone would cost up to 2^-9 of max|v| when a few
// keys dominate).
template <int KV>
__device__ __forceinline__ void pack8_split(const float (&p)[8], u32x4& hi, u32x4& lo) {
  if constexpr (KV == kF16) {
    f16x8 h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = (_Float16)p[e];
      l[e] = (_Float16)(p[e] - (float)h[e]);
    }
    hi = __builtin_bit_cast(u32x4, h);
    lo = __builtin_bit_cast(u32x4, l);
  } else {
    bf16x8 h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = (__bf16)p[e];
      l[e] = (__bf16)(p[e] - (float)h[e]);
    }
    hi = __builtin_bit_cast(u32x4, h);
    lo = __builtin_bit_cast(u32x4, l);
  }
}

__device__ __forceinline__ float xor_max(float v, int m) {
  return fmaxf(v, __shfl_xor(v, m, kWave));
}

// Per-sequence decode shared by both kernels: the contract check and the
// step/segment ranges.  Keys of the sequence that any row reads lie in
// [lo0, ctx); steps are kKeysPerStep-key windows starting at base.
struct SeqInfo {
  int b0, T, L, ctx, lo0, base, n_steps;
  bool ok;
};

__device__ __forceinline__ SeqInfo seq_info(const SegmentArgs& a, int s) {
  SeqInfo q;
  q.b0 = a.sb[s];
  const int b1 = a.sb[s + 1];
  q.T = b1 - q.b0;
  q.L = a.past_lens[s];
  q.ok = q.b0 >= 0 && b1 <= a.num_tokens && q.T >= 1 && q.T <= kMaxT && q.L >= 0 &&
         (int64_t)q.L + q.T <= a.max_ctx && a.G * q.T <= kRows;
  q.ctx = q.L + q.T;
  q.lo0 = a.window > 0 ? max(0, q.L + 1 - a.window) : 0;
  q.base = (q.lo0 / kKeysPerStep) * kKeysPerStep;
  q.n_steps = q.ok ? (q.ctx - q.base + kKeysPerStep - 1) / kKeysPerStep : 0;
  return q;
}

// ---------------------------------------------------------------------------
// Segment kernel, f16 / bf16 KV.
// ---------------------------------------------------------------------------
template <int KV, int D, int BS, int NW, int WPE>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(WPE)))
void pa_segment_fp(SegmentArgs a) {
  constexpr int DC = D / 32;          // 32-wide d chunks of the QK contraction
  constexpr int DT = D / 16;          // 16-wide d tiles of O^T
  constexpr int OSTRIDE = D + 4;      // padded LDS row of the merge buffer
  __shared__ int s_bt[kMaxSegBlocks];
  __shared__ float s_m[NW][kRows];
  __shared__ float s_l[NW][kRows];
  __shared__ __attribute__((aligned(16))) float s_o[NW][kRows][OSTRIDE];
  __shared__ int s_bad;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n16 = lane & 15;          // stacked query row owned by this lane
  const int q4 = lane >> 4;           // lane group: 8 keys of a step, 8 d of a chunk
  const int j = blockIdx.x, h = blockIdx.y, s = blockIdx.z;

  const SeqInfo si = seq_info(a, s);
  if (!si.ok) {
    if (j == 0 && h == 0 && threadIdx.x == 0) atomicExch(a.status, kDeviceContract);
    return;                           // the combine kernel writes NaN rows
  }
  const int st_begin = j * a.steps_per_seg;
  const int st_end = min(si.n_steps, st_begin + a.steps_per_seg);
  if (st_begin >= st_end) return;     // empty segment; the combine skips it

  // Stage the segment's block ids in LDS.  Only pages holding a key in
  // [lo0, ctx) are checked and ever dereferenced.
  const int key_lo = si.base + st_begin * kKeysPerStep;
  const int blk_lo = key_lo / BS;
  const int blk_last = (min(si.ctx, si.base + st_end * kKeysPerStep) - 1) / BS;
  const int32_t* bt_row = a.bt + (size_t)s * a.mbps;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  for (int x = threadIdx.x; x <= blk_last - blk_lo; x += NW * kWave) {
    const int b = blk_lo + x;
    int id = 0;
    if ((b + 1) * BS > si.lo0) {
      id = bt_row[b];
      if ((unsigned)id >= (unsigned)a.num_blocks) {
        s_bad = 1;
        id = 0;
      }
    }
    s_bt[x] = id;
  }

  // Stacked rows: r = g*T + i for q head h*G + g and token b0 + i; rows past
  // G*T are zero padding that no one reads back.
  const int T = si.T;
  const int R = a.G * T;
  const bool row_ok = n16 < R;
  const int g = row_ok ? n16 / T : 0;
  const int i = row_ok ? n16 % T : T - 1;
  const int qh = h * a.G + g;
  const int tok = si.b0 + i;
  const int hi_r = si.L + i + 1;                              // row's keys: [lo_r, hi_r)
  const int lo_r = a.window > 0 ? max(0, hi_r - a.window) : 0;
  const int lo_max = a.window > 0 ? max(0, si.ctx - a.window) : 0;

  u32x4 qreg[DC];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) + (((size_t)tok * a.Hq + qh) * D + q4 * 8) * 2;
#pragma unroll
    for (int c = 0; c < DC; ++c) qreg[c] = row_ok ? ld16(qp + c * 64) : u32x4{0, 0, 0, 0};
  }
  __syncthreads();

  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  const size_t tile_elems = (size_t)BS * D;                   // one (block, head) page
  const int Hkv = a.Hkv;

  // Registers of one step: K rows for two 16-key QK tiles, V^T for DT d tiles.
  auto load_step = [&](int st, u32x4 (&kr)[2][DC], u32x4 (&vr)[DT]) {
    const int key0 = si.base + st * kKeysPerStep;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      // QK tile tau: A row m = n16 holds step key (m/4)*8 + tau*4 + m%4, so
      // the output lands in lane group q4 as keys q4*8 + tau*4 + (0..3).
      const int t = key0 + (n16 >> 2) * 8 + tau * 4 + (n16 & 3);
      const bool present = t >= si.lo0 && t < si.ctx;
      const int phys = present ? s_bt[t / BS - blk_lo] : 0;
      const char* p = kb + (((size_t)phys * Hkv + h) * tile_elems + (size_t)(t % BS) * D + q4 * 8) * 2;
#pragma unroll
      for (int c = 0; c < DC; ++c) kr[tau][c] = present ? ld16(p + c * 64) : u32x4{0, 0, 0, 0};
    }
    const int tv = key0 + q4 * 8;                             // this lane's 8 keys
    const bool vpresent = tv < si.ctx && tv + 8 > si.lo0;
    const int physv = vpresent ? s_bt[tv / BS - blk_lo] : 0;
    const char* pv = vb + (((size_t)physv * Hkv + h) * tile_elems + (size_t)n16 * BS + (tv % BS)) * 2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vr[dt] = vpresent ? ld16(pv + (size_t)dt * 16 * BS * 2) : u32x4{0, 0, 0, 0};
  };

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;            // running max (log2 units) of this lane's row
  float l_run = 0.f;                  // this lane's share of the running sum

  auto compute_step = [&](int st, u32x4 (&kr)[2][DC], u32x4 (&vr)[DT]) {
    const int key0 = si.base + st * kKeysPerStep;
    f32x4 sacc[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      sacc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) sacc[tau] = mfma32<KV>(kr[tau][c], qreg[c], sacc[tau]);
    }
    float sv[8];                      // keys key0 + q4*8 + e of row n16
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = sacc[e >> 2][e & 3] * a.scale_log2;

    const bool interior = key0 >= lo_max && key0 + kKeysPerStep <= si.L + 1;
    if (!interior) {
      const int t0 = key0 + q4 * 8;
      uint32_t keep[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int ta = t0 + 2 * w, tb = ta + 1;
        keep[w] = ((ta >= si.lo0 && ta < si.ctx) ? 0x0000FFFFu : 0u) |
                  ((tb >= si.lo0 && tb < si.ctx) ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + e;
        sv[e] = (t >= lo_r && t < hi_r) ? sv[e] : -INFINITY;
      }
      // keys outside the sequence's readable range may hold anything, NaN
      // included; their weight is 0 but 0 * NaN is not, so clear them
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        vr[dt][0] &= keep[0];
        vr[dt][1] &= keep[1];
        vr[dt][2] &= keep[2];
        vr[dt][3] &= keep[3];
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
      psum += p[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4 pb_hi, pb_lo;
    pack8_split<KV>(p, pb_hi, pb_lo);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] *= alpha;
      o[dt] = mfma32<KV>(vr[dt], pb_hi, o[dt]);
      o[dt] = mfma32<KV>(vr[dt], pb_lo, o[dt]);
    }
  };

  {
    int st = st_begin + wave;
    u32x4 kr[2][DC], vr[DT];
    if (st < st_end) load_step(st, kr, vr);
    while (st < st_end) {
      const int nx = st + NW;
      u32x4 kn[2][DC], vn[DT];
      if (nx < st_end) load_step(nx, kn, vn);
      compute_step(st, kr, vr);
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int c = 0; c < DC; ++c) kr[tau][c] = kn[tau][c];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vr[dt] = vn[dt];
      st = nx;
    }
  }

  // Row sums: each lane group holds a quarter of the keys.
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);

  // Merge the wavefronts of the workgroup: M = max_w m_w, then sum the
  // partials rescaled by 2^(m_w - M), in a fixed order (bitwise repeatable).
  if (q4 == 0) {
    s_m[wave][n16] = m_run;
    s_l[wave][n16] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4*>(&s_o[wave][n16][dt * 16 + q4 * 4]) = o[dt];
  __syncthreads();

  const bool bad = s_bad != 0;
  constexpr int V4 = D / 4;                                   // float4 columns per row
  for (int x = threadIdx.x; x < R * V4; x += NW * kWave) {
    const int r = x / V4;
    const int c4 = (x % V4) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][r]);
    const int rt = si.b0 + r % T;
    const int rh = h * a.G + r / T;
    const size_t row = ((size_t)rt * a.Hq + rh) * a.S + j;   // partials are per token
    if (M == -INFINITY) {                                     // no key of this row here
      if (c4 == 0) {
        a.ws_ml[row * 2 + 0] = bad ? NAN : -INFINITY;
        a.ws_ml[row * 2 + 1] = 0.f;
      }
      continue;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w][r] - M);
      acc += f * *reinterpret_cast<const f32x4*>(&s_o[w][r][c4]);
      lsum += f * s_l[w][r];
    }
    *reinterpret_cast<f32x4*>(&a.ws_o[row * D + c4]) = acc;
    if (c4 == 0) {
      a.ws_ml[row * 2 + 0] = bad ? NAN : M;
      a.ws_ml[row * 2 + 1] = lsum;
    }
  }
  if (bad && threadIdx.x == 0) atomicExch(a.status, kDeviceContract);
}

// ---------------------------------------------------------------------------
// Combine kernel: one workgroup per (token, q head).  Thread t owns d columns
// [c4, c4 + 4) of the segments sub, sub + NSUB, ...; it merges them with the
// same online rescaling as the segment kernel (every load independent of the
// previous iteration's arithmetic, so they all go out at once), then the
// NSUB partial states are merged through LDS in a fixed order.
// ---------------------------------------------------------------------------
template <int D, int OUT>
__global__ __launch_bounds__(256) void pa_combine(CombineArgs a) {
  constexpr int LPS = D / 4;                                  // threads per segment row
  constexpr int NSUB = 256 / LPS;                             // segment rows in flight
  __shared__ float s_m[NSUB];
  __shared__ float s_den[NSUB];
  __shared__ __attribute__((aligned(16))) f32x4 s_acc[NSUB][LPS];

  const int pair = blockIdx.x;                                // token * Hq + q head
  const int tid = threadIdx.x;
  const int sub = tid / LPS;
  const int col = tid % LPS;
  const int n = pair / a.Hq;

  // sequence of token n (subsequence_begins is cumulative)
  int s = 0;
  while (s < a.seg.num_seqs && !(n < a.seg.sb[s + 1])) ++s;
  bool ok = s < a.seg.num_seqs && n >= a.seg.sb[s];
  int n_seg = 0;
  if (ok) {
    const SeqInfo si = seq_info(a.seg, s);
    ok = si.ok;
    n_seg = min(a.seg.S, (si.n_steps + a.seg.steps_per_seg - 1) / a.seg.steps_per_seg);
  }
  const float* ml = a.seg.ws_ml + (size_t)pair * a.seg.S * 2;
  const float* op = a.seg.ws_o + (size_t)pair * a.seg.S * D + col * 4;
  float m = -INFINITY, den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bool nan_seen = false;
#pragma unroll 4
  for (int jj = sub; jj < n_seg; jj += NSUB) {
    const float mj = ml[jj * 2];
    const float lj = ml[jj * 2 + 1];
    const f32x4 oj = *reinterpret_cast<const f32x4*>(op + (size_t)jj * D);
    nan_seen |= mj != mj;
    const float m_new = fmaxf(m, mj);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float sc = __builtin_amdgcn_exp2f(m - base);
    const float f = __builtin_amdgcn_exp2f(mj - base);
    den = den * sc + f * lj;
    // a segment in which this row saw no key left its O slot unwritten
    acc = mj == -INFINITY ? acc * sc : acc * sc + f * oj;
    m = m_new;
  }
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

// ---------------------------------------------------------------------------
// Instances and launchers.
// ---------------------------------------------------------------------------
template <int KV, int D, int BS>
static hipError_t launch_segment_fp(const SegmentArgs& a, dim3 grid, hipStream_t st,
                                    hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int WPE = D >= 256 ? 1 : (D >= 128 ? 2 : 4);
  // with events, the dispatch itself timestamps the kernel's start and end
  if (ev0 || ev1)
    hipExtLaunchKernelGGL((pa_segment_fp<KV, D, BS, kWavesPerGroup, WPE>), grid,
                          dim3(kWavesPerGroup * kWave), 0, st, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL((pa_segment_fp<KV, D, BS, kWavesPerGroup, WPE>), grid,
                       dim3(kWavesPerGroup * kWave), 0, st, a);
  return hipGetLastError();
}

template <int KV, int D>
static hipError_t dispatch_bs(const SegmentArgs& a, int bs, dim3 grid, hipStream_t st,
                              hipEvent_t e0, hipEvent_t e1) {
  switch (bs) {
    case 16: return launch_segment_fp<KV, D, 16>(a, grid, st, e0, e1);
    case 32: return launch_segment_fp<KV, D, 32>(a, grid, st, e0, e1);
    case 64: return launch_segment_fp<KV, D, 64>(a, grid, st, e0, e1);
  }
  return hipErrorInvalidValue;
}

template <int KV>
static hipError_t dispatch_d(const SegmentArgs& a, int D, int bs, dim3 grid, hipStream_t st,
                             hipEvent_t e0, hipEvent_t e1) {
  switch (D) {
    case 64: return dispatch_bs<KV, 64>(a, bs, grid, st, e0, e1);
    case 128: return dispatch_bs<KV, 128>(a, bs, grid, st, e0, e1);
    case 256: return dispatch_bs<KV, 256>(a, bs, grid, st, e0, e1);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_segment(const SegmentArgs& a, int kv_dtype, int D, int bs, dim3 grid,
                          hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  if (kv_dtype == kF16) return dispatch_d<kF16>(a, D, bs, grid, st, e0, e1);
  if (kv_dtype == kBF16) return dispatch_d<kBF16>(a, D, bs, grid, st, e0, e1);
  return hipErrorInvalidValue;
}

hipError_t launch_segment_u8(const SegmentArgs&, int, int, int, dim3, hipStream_t, hipEvent_t,
                             hipEvent_t) {
  return hipErrorNotSupported;
}

template <int D>
static hipError_t launch_combine_d(const CombineArgs& a, int out_dtype, dim3 grid, hipStream_t st) {
  if (out_dtype == kF16)
    hipLaunchKernelGGL((pa_combine<D, kF16>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((pa_combine<D, kBF16>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int out_dtype, int D, dim3 grid, hipStream_t st) {
  switch (D) {
    case 64: return launch_combine_d<64>(a, out_dtype, grid, st);
    case 128: return launch_combine_d<128>(a, out_dtype, grid, st);
    case 256: return launch_combine_d<256>(a, out_dtype, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pav
