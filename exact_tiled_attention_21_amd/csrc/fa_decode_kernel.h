// Split-KV attention for decode (Flash-Decoding) on gfx950.
//
// "flash-attention-v100" README, Changelog 2.2: with very short query blocks
// the cost is reading the KV cache, so the key range is split over several
// workgroups and a separate kernel merges the results. The "flash attention-2
// github" search page spells out the steps: split K/V into chunks, attend to
// every chunk in parallel while writing one extra scalar per row and chunk
// (the log-sum-exp), then combine.
//
// Split kernel: one workgroup per (chunk, KV head, batch[, row block]). The
// query rows of the whole GQA group (Hq/Hkv heads x Nq positions, at most 32
// per row block) share the chunk's K/V, which is therefore read from HBM once.
// The four waves take interleaved 32-key tiles of the chunk. K fragments are
// loaded straight from global memory into MFMA A-operand registers (no LDS);
// V tiles go through a small wave-private, swizzled LDS tile so the
// transposing read can build the V^T operand. Loads of a wave's next tile are
// issued before the current one is consumed. The four waves' (max, sum, O)
// states are merged through LDS and written as one normalised fp32 partial and
// its log-sum-exp per row.
//
// Combine kernel: per output row, LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s; chunks with LSE_s = -inf weigh nothing.
#pragma once

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D> struct DecCfg {
  static constexpr int NW = 4;
  static constexpr int THREADS = NW * 64;
  static constexpr int BC = 32;                 // keys per wave tile
  static constexpr int NS = D / 16;
  static constexpr int NCB = D / 32;
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int VCPL = BC * CPR / 64;    // V chunks per lane per tile
  static constexpr int VTILE = BC * D * 2;      // bytes of one wave's V tile
  static constexpr int MERGE = (NW - 1) * (NCB * 16 + 2) * 64 * 4;  // published wave states
  static constexpr int LDS_BYTES = (NW * VTILE > MERGE) ? NW * VTILE : MERGE;
};

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_decode_split_kernel(const DecodeArgs a) {
  using C = DecCfg<D>;
  using E = Elem<BF16>;
  using T = typename E::T;
  using V8 = typename E::V8;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  const int split = blockIdx.x;
  const int g = blockIdx.y % a.Hkv;
  const int rb = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int R = a.group * a.Nq;             // rows of this KV head group
  const int diag = a.Nk - a.Nq;

  // row r = i * group + (hq - g * group): consecutive rows are adjacent heads
  const int r = rb * 32 + (lane & 31);
  const bool rvalid = r < R;
  const int ri = rvalid ? r / a.group : 0;
  const int rhq = g * a.group + (rvalid ? r % a.group : 0);

  V8 qf[C::NS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) +
                  ((static_cast<size_t>(b) * a.Nq + ri) * a.Hq + rhq) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      if (rvalid) qf[s] = *reinterpret_cast<const V8*>(qp + 16 * s);
      else qf[s] = V8{};
    }
  }

  // keys of this chunk, clipped by the cache length and (causal) the last row
  const int k_lo = split * a.chunk;
  int k_hi = min(a.Nk, k_lo + a.chunk);
  int i_first = (rb * 32) / a.group;                    // smallest query position
  if (CAUSAL) {
    const int i_last = (min(R, rb * 32 + 32) - 1) / a.group;
    k_hi = min(k_hi, i_last + diag + 1);
  }
  const int ntile = k_hi > k_lo ? (k_hi - k_lo + C::BC - 1) / C::BC : 0;

  const size_t rstride = static_cast<size_t>(a.Hkv) * D;
  const T* kbase = reinterpret_cast<const T*>(a.k) + (static_cast<size_t>(b) * a.Nk * a.Hkv + g) * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (static_cast<size_t>(b) * a.Nk * a.Hkv + g) * D;
  char* vt = smem + wave * C::VTILE;

  V8 kf[C::NS];
  u32x4 vst[C::VCPL];
  auto gload = [&](int tile) {
    const int key = k_lo + tile * C::BC + (lane & 31);
    const bool ok = key < k_hi;
    const T* kp = kbase + static_cast<size_t>(ok ? key : 0) * rstride + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) kf[s] = ok ? *reinterpret_cast<const V8*>(kp + 16 * s) : V8{};
#pragma unroll
    for (int i = 0; i < C::VCPL; ++i) {
      const int c = lane + 64 * i;
      const int vkey = k_lo + tile * C::BC + c / C::CPR;
      vst[i] = vkey < k_hi ? *reinterpret_cast<const u32x4*>(vbase + static_cast<size_t>(vkey) * rstride + 8 * (c % C::CPR))
                           : u32x4{0, 0, 0, 0};
    }
  };

  f32x16 oacc[C::NCB];
#pragma unroll
  for (int cb = 0; cb < C::NCB; ++cb) oacc[cb] = f32x16{};
  float m_run = kNegInf, l_part = 0.f;

  int tile = wave;
  if (tile < ntile) gload(tile);
  for (; tile < ntile; tile += C::NW) {
    // stage V of this tile; the current K fragment moves out of the prefetch registers
    V8 kc[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) kc[s] = kf[s];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < C::VCPL; ++i) {
      const int c = lane + 64 * i;
      *reinterpret_cast<u32x4*>(vt + Swz<D>::off(c / C::CPR, c % C::CPR)) = vst[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (tile + C::NW < ntile) gload(tile + C::NW);

    const int k0 = k_lo + tile * C::BC;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < C::NS; ++s) sacc = E::mfma(kc[s], qf[s], sacc);
    const bool need_mask = (k0 + C::BC > k_hi) || (CAUSAL && k0 + C::BC - 1 > i_first + diag);
    float mx = kNegInf;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float x = sacc[q] * a.sl2;
      if (need_mask) {
        const int key = k0 + 8 * (q >> 2) + 4 * hh + (q & 3);
        if (key >= k_hi || (CAUSAL && key > ri + diag)) x = kNegInf;
      }
      sacc[q] = x;
      mx = fmaxf(mx, x);
    }
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float p = exp2_fast(sacc[q] - m_use);
      sacc[q] = p;
      psum += p;
    }
    l_part = l_part * alpha + psum;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) oacc[cb] *= alpha;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const V8 pf = to_v8<BF16>(sacc, 8 * t);
#pragma unroll
      for (int cb = 0; cb < C::NCB; ++cb) oacc[cb] = E::mfma(v_frag<D, V8>(vt, cb, t, lane), pf, oacc[cb]);
    }
  }

  // merge the waves: all of them hold (row, column) at the same lane and
  // register, so waves 1..3 publish their raw state lane-major and wave 0
  // folds it into its own registers
  __syncthreads();  // every wave is done with its V tile
  constexpr int NV = C::NCB * 16;                          // O values per lane
  float* pub = reinterpret_cast<float*>(smem);             // [NW-1][NV+2][64]
  if (wave > 0) {
    float* mine = pub + (wave - 1) * (NV + 2) * 64 + lane;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
      for (int q = 0; q < 16; ++q) mine[(cb * 16 + q) * 64] = oacc[cb][q];
    mine[NV * 64] = m_run;
    mine[(NV + 1) * 64] = l_part;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < C::NW; ++w) {
    const float* other = pub + (w - 1) * (NV + 2) * 64 + lane;
    const float m_o = other[NV * 64];
    const float m_new = fmaxf(m_run, m_o);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float a0 = exp2_fast(m_run - m_use), a1 = exp2_fast(m_o - m_use);
    l_part = l_part * a0 + other[(NV + 1) * 64] * a1;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
      for (int q = 0; q < 16; ++q) oacc[cb][q] = oacc[cb][q] * a0 + other[(cb * 16 + q) * 64] * a1;
    m_run = m_new;
  }
  const float l = halves_sum(l_part);
  if (!rvalid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t prow = ((static_cast<size_t>(split) * a.B + b) * a.Hq + rhq) * a.Nq + ri;
  float* po = a.part_o + prow * D;
#pragma unroll
  for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
    for (int gr = 0; gr < 4; ++gr) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = oacc[cb][4 * gr + e] * inv;
      *reinterpret_cast<f32x4*>(po + 32 * cb + 8 * gr + 4 * hh) = w;
    }
  if (hh == 0) a.part_lse[prow] = l > 0.f ? m_run + __log2f(l) : kNegInf;
}

// One row of the output per D/4 threads: O = sum_s w_s O_s with
// w_s = exp(LSE_s - LSE), LSE = log sum_s exp(LSE_s) (log2 domain inside).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void fa_decode_combine_kernel(const DecodeArgs a) {
  using T = typename Elem<BF16>::T;
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int rows = a.B * a.Hq * a.Nq;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c4 = (threadIdx.x % TPR) * 4;
  const size_t stride = static_cast<size_t>(rows);   // elements between splits
  float mx = kNegInf;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.part_lse[s * stride + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (mx != kNegInf) {
    for (int s = 0; s < a.splits; ++s) {
      const float w = exp2_fast(a.part_lse[s * stride + row] - mx);
      tot += w;
      acc += w * *reinterpret_cast<const f32x4*>(a.part_o + (s * stride + row) * D + c4);
    }
    acc *= 1.f / tot;
  }
  // row = (b * Hq + hq) * Nq + i  ->  o[b][i][hq][:]
  const int i = row % a.Nq;
  const int bh = row / a.Nq;
  const int hq = bh % a.Hq;
  const int b = bh / a.Hq;
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (T)acc[e];
  *reinterpret_cast<T4*>(reinterpret_cast<T*>(a.o) + ((static_cast<size_t>(b) * a.Nq + i) * a.Hq + hq) * D + c4) = w;
  if (a.lse != nullptr && c4 == 0) a.lse[row] = (mx == kNegInf) ? kNegInf : (mx + __log2f(tot)) * kLn2;
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, bool bf16, bool causal, hipStream_t stream) {
  using C = DecCfg<D>;
  const dim3 grid1(a.splits, a.Hkv * a.row_blocks, a.B);
  const void* f1 = bf16 ? (causal ? (const void*)fa_decode_split_kernel<D, true, true>
                                  : (const void*)fa_decode_split_kernel<D, true, false>)
                        : (causal ? (const void*)fa_decode_split_kernel<D, false, true>
                                  : (const void*)fa_decode_split_kernel<D, false, false>);
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  if (C::LDS_BYTES > 65536) {
    hipError_t e = hipFuncSetAttribute(f1, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipLaunchKernel(f1, grid1, dim3(C::THREADS), args, C::LDS_BYTES, stream);
  if (e != hipSuccess) return e;
  constexpr int RPB = 256 / (D / 4);
  const int rows = a.B * a.Hq * a.Nq;
  const dim3 grid2((rows + RPB - 1) / RPB);
  const void* f2 = bf16 ? (const void*)fa_decode_combine_kernel<D, true> : (const void*)fa_decode_combine_kernel<D, false>;
  return hipLaunchKernel(f2, grid2, dim3(256), args, 0, stream);
}

}  // namespace fa
