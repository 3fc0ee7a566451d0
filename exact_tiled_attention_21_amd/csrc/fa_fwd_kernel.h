// Exact attention forward kernel (FlashAttention-2 work partitioning) for gfx950.
//
// Parallel over (query tile, head, batch): the "Flash attention gpu" page
// notes that batch and heads are independent and that different query blocks
// are independent too, so each workgroup owns 128 query rows of one head and
// loops over all key/value tiles ("flash-attention-v100" README: FlashAttention-2
// reworked the parallelism and work partitioning). Four waves of 32 rows each;
// the Q fragment stays in VGPRs for the whole loop; K/V tiles are staged
// through a double-buffered, XOR-swizzled LDS ring so the loads of tile j+1
// are in flight while tile j is consumed; the online softmax keeps a running
// max and sum per row and rescales the O accumulator, so the Nq x Nk scores
// never leave registers.
#pragma once

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D> struct FwdCfg {
  static constexpr int NW = 4;                       // waves per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int BR = 32 * NW;                 // query rows per workgroup
  static constexpr int BC = (D <= 128) ? 64 : 32;    // keys per LDS tile
  static constexpr int KB = BC / 32;                 // 32-key blocks of S^T
  static constexpr int NS = D / 16;                  // 16-wide d slices (QK^T depth)
  static constexpr int NCB = D / 32;                 // 32-wide d blocks of O^T
  static constexpr int NT = BC / 16;                 // 16-key slices (PV depth)
  static constexpr int TILE_BYTES = BC * D * 2;
  static constexpr int LDS_BYTES = 2 * 2 * TILE_BYTES;  // 2 stages x (K, V)
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / THREADS;     // chunks per thread per tensor
  static_assert(BR == kFwdRows, "rows per workgroup");
  static_assert(BC * CPR % THREADS == 0, "tile must split evenly over threads");
};

template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_fwd_kernel(const FwdArgs a) {
  using C = FwdCfg<D>;
  using E = Elem<BF16>;
  using T = typename E::T;
  using V8 = typename E::V8;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;

  // workgroup -> (query tile, head, batch)
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int qt = bid % a.n_qtiles;
  const int hb = bid / a.n_qtiles;
  const int hq = hb % a.Hq;
  const int b = hb / a.Hq;
  if (CAUSAL) qt = a.n_qtiles - 1 - qt;  // longest rows first
  const int g = hq / a.group;

  const int q0w = qt * C::BR + wave * 32;   // first row of this wave
  const int qrow = q0w + (lane & 31);       // this lane's query row
  const int diag = a.Nk - a.Nq;             // query i sees key j iff j <= i + diag

  // Q fragment (B operand): Q[qrow][16s + 8hh .. +7]
  V8 qf[C::NS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) +
                  ((static_cast<size_t>(b) * a.Nq + qrow) * a.Hq + hq) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      if (qrow < a.Nq) qf[s] = *reinterpret_cast<const V8*>(qp + 16 * s);
      else qf[s] = V8{};
    }
  }

  // key extents: the workgroup loads tiles up to kend; this wave computes up to wkend
  int kend = a.Nk, wkend = a.Nk;
  {
    const int last_wg = min(qt * C::BR + C::BR, a.Nq) - 1;
    const int last_w = min(q0w + 32, a.Nq) - 1;
    if (CAUSAL) {
      kend = min(a.Nk, last_wg + diag + 1);
      wkend = min(a.Nk, last_w + diag + 1);
    }
    if (q0w >= a.Nq) wkend = 0;
  }
  const int ntiles = kend > 0 ? (kend + C::BC - 1) / C::BC : 0;

  // global -> register staging of one K and one V tile
  const T* kbase = reinterpret_cast<const T*>(a.k) + (static_cast<size_t>(b) * a.Nk * a.Hkv + g) * D;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (static_cast<size_t>(b) * a.Nk * a.Hkv + g) * D;
  const size_t rstride = static_cast<size_t>(a.Hkv) * D;
  u32x4 kst[C::CPT], vst[C::CPT];
  auto gload = [&](int tile) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::THREADS;
      const int row = c / C::CPR, x = c % C::CPR;
      const int key = tile * C::BC + row;
      if (key < a.Nk) {
        kst[i] = *reinterpret_cast<const u32x4*>(kbase + key * rstride + 8 * x);
        vst[i] = *reinterpret_cast<const u32x4*>(vbase + key * rstride + 8 * x);
      } else {
        kst[i] = u32x4{0, 0, 0, 0};
        vst[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int stage) {
    char* kt = smem + stage * 2 * C::TILE_BYTES;
    char* vt = kt + C::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::THREADS;
      const uint32_t o = Swz<D>::off(c / C::CPR, c % C::CPR);
      *reinterpret_cast<u32x4*>(kt + o) = kst[i];
      *reinterpret_cast<u32x4*>(vt + o) = vst[i];
    }
  };

  f32x16 oacc[C::NCB];
#pragma unroll
  for (int cb = 0; cb < C::NCB; ++cb) oacc[cb] = f32x16{};
  float m_run = kNegInf;  // running max of scale*log2(e)*s
  float l_part = 0.f;     // running sum over this lane's keys

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int stage = j & 1;
    if (j + 1 < ntiles) gload(j + 1);
    const int k0 = j * C::BC;
    if (k0 < wkend) {
      const char* kt = smem + stage * 2 * C::TILE_BYTES;
      const char* vt = kt + C::TILE_BYTES;
      // S^T = K Q^T
      f32x16 sacc[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < C::NS; ++s) sacc[kb] = E::mfma(k_frag<D, V8>(kt, kb, s, lane), qf[s], sacc[kb]);
      }
      // scale, mask, row max
      const bool need_mask = (k0 + C::BC > a.Nk) || (CAUSAL && k0 + C::BC - 1 > q0w + diag);
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kb][r] * a.sl2;
          if (need_mask) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= a.Nk || (CAUSAL && key > qrow + diag)) x = kNegInf;
          }
          sacc[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = halves_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(sacc[kb][r] - m_use);
          sacc[kb][r] = p;
          psum += p;
        }
      }
      l_part = l_part * alpha + psum;
#pragma unroll
      for (int cb = 0; cb < C::NCB; ++cb) oacc[cb] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        const V8 pf = to_v8<BF16>(sacc[t >> 1], 8 * (t & 1));
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb) oacc[cb] = E::mfma(v_frag<D, V8>(vt, cb, t, lane), pf, oacc[cb]);
      }
    }
    if (j + 1 < ntiles) lstore(stage ^ 1);
    __syncthreads();
  }

  // epilogue: O = O / l, LSE = m + log(l); rows with no visible key give 0 and -inf
  const float l = halves_sum(l_part);
  if (qrow < a.Nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    T* op = reinterpret_cast<T*>(a.o) + ((static_cast<size_t>(b) * a.Nq + qrow) * a.Hq + hq) * D;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) {
#pragma unroll
      for (int gr = 0; gr < 4; ++gr) {
        typedef T T4 __attribute__((ext_vector_type(4)));
        T4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (T)(oacc[cb][4 * gr + e] * inv);
        *reinterpret_cast<T4*>(op + 32 * cb + 8 * gr + 4 * hh) = w;
      }
    }
    if (a.lse != nullptr && hh == 0)
      a.lse[(static_cast<size_t>(b) * a.Hq + hq) * a.Nq + qrow] =
          l > 0.f ? (m_run + __log2f(l)) * kLn2 : kNegInf;
  }
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, bool bf16, bool causal, hipStream_t stream) {
  using C = FwdCfg<D>;
  const dim3 grid(static_cast<unsigned>(a.n_qtiles) * a.Hq * a.B);
  const dim3 block(C::THREADS);
  const void* fn = bf16 ? (causal ? (const void*)fa_fwd_kernel<D, true, true> : (const void*)fa_fwd_kernel<D, true, false>)
                        : (causal ? (const void*)fa_fwd_kernel<D, false, true> : (const void*)fa_fwd_kernel<D, false, false>);
  void* args[] = {const_cast<FwdArgs*>(&a)};
  return hipLaunchKernel(fn, grid, block, args, C::LDS_BYTES, stream);
}

}  // namespace fa
