// Register-staged forward kernel (gfx950): the path for fp32 Q/K/V, which
// are rounded to bf16 (RNE) as they are loaded.
//
// Same walk and arithmetic as the DMA kernel in bsa_fwd.hip, but each 64-key
// K/V sub-tile passes through registers: the next sub-tile's rows are loaded
// and converted while the current one computes, then written to the other
// LDS stage, K row-major and V transposed (V^T[d][key]) so both MFMA A
// operands are 16-byte LDS reads.
//
// The PROXY instance adds the proxy-compensated route of the PrimTS page
// ("proxy-compensated block-sparse attention", flashinfer pull request 4872):
// after the listed blocks, the same pipeline walks the caller's block
// summaries 64 at a time as if they were keys (mean K as the key, summed V
// as the value).  An LDS bitmap of the Q block's listed blocks masks the
// summaries of blocks that are attended exactly, chunks whose blocks are all
// listed are skipped, and the row sum counts each summary at its block's
// token mass, so the result is one softmax over exact keys and proxies.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bsa_fwd_common.h"
#include "bsa_fwd_proxy.h"

namespace bsa {
namespace {

using namespace dev;

// 8 consecutive input elements as 8 bf16.
template <bool F32> struct Chunk;
template <> struct Chunk<false> {
  uint4 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
};
template <> struct Chunk<true> {
  uint4 v;
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                   pack_bf16x2(b.z, b.w));
  }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int D, int NW, bool F32IN, bool PROXY>
__global__ __launch_bounds__(NW * 64) void bsa_fwd_staged_kernel(const FwdParams p) {
  using T = typename std::conditional<F32IN, float, __bf16>::type;
  constexpr int NT = NW * 64;
  constexpr int TM = NW * 32;
  constexpr int KT = kKvTile;
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  constexpr int KROW = D * 2 + 16;   // LDS bytes per K row (16 B pad)
  constexpr int VROW = KT * 2 + 16;  // LDS bytes per V^T row (16 B pad)
  constexpr int KBYTES = KT * KROW;
  constexpr int STAGE = KBYTES + D * VROW;
  constexpr int DC = D / 8;
  constexpr int KCH = KT * DC;
  constexpr int KC = (KCH + NT - 1) / NT;
  constexpr int VBL = (KT / 4) * DC;  // 4-key x 8-dim V blocks per sub-tile
  constexpr int VB = (VBL + NT - 1) / NT;
  static_assert(D % 32 == 0, "head_dim must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];
  // listed blocks of this Q block (+1 word: a chunk's second word may lie past the last)
  __shared__ uint32_t xbits[PROXY ? kProxyBitmapWords : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, l32 = lane & 31, h32 = lane >> 5;

  TileInfo ti;
  const int tix = xcd_remap(blockIdx.x, p.num_tiles);
  if (!decode_tile<TM>(p, tix, ti)) return;
  const T* qp = reinterpret_cast<const T*>(p.q) + ti.qoff;
  const T* kp = reinterpret_cast<const T*>(p.k) + ti.koff;
  const T* vp = reinterpret_cast<const T*>(p.v) + ti.voff;
  const T* ksp = nullptr;
  const T* vsp = nullptr;
  if constexpr (PROXY) {  // batched only: tile = ((b*H + h) * tiles_per_head + qt)
    const int bh = tix / p.tiles_per_head;
    const int b = bh / p.H, hk = (bh % p.H) / p.hrep;
    ksp = reinterpret_cast<const T*>(p.ksum) + b * p.ks_sb + hk * p.ks_sh;
    vsp = reinterpret_cast<const T*>(p.vsum) + b * p.vs_sb + hk * p.vs_sh;
    build_listed_bitmap(xbits, p, ti, tid, NT);
  }

  const int qrow = ti.q0 + 32 * w + l32;
  const bool live = ti.q0 + 32 * w < ti.qend;  // else only stage and wait (rows past the block)
  uint4 qf[DS];
#pragma unroll
  for (int ks = 0; ks < DS; ++ks) {
    Chunk<F32IN> c;
    if (qrow < ti.qend)
      c.load(qp + (int64_t)qrow * p.q_ss + ks * 16 + h32 * 8);
    else
      c.zero();
    qf[ks] = c.v;
  }
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = neg_inf(), l_run = 0.f, lo_run = 0.f;

  Chunk<F32IN> kst[KC];
  Chunk<F32IN> vst[VB][4];
  auto issue = [&](const Item& it) {
    const bool px = PROXY && it.is_mask == 2;
    const T* kb = px ? ksp : kp;
    const T* vb_ = px ? vsp : vp;
    const int64_t kss = px ? p.ks_ss : p.k_ss;
    const int64_t vss = px ? p.vs_ss : p.v_ss;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int ci = tid + c * NT;
      if (KCH % NT == 0 || ci < KCH) {
        const int row = ci / DC, col = ci % DC;
        if (row < it.nk)
          kst[c].load(kb + (int64_t)(it.key0 + row) * kss + col * 8);
        else
          kst[c].zero();
      }
    }
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int bi = tid + vb * NT;
      if (VBL % NT == 0 || bi < VBL) {
        const int kg = bi / DC, dc = bi % DC;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = kg * 4 + rr;
          if (key < it.nk)
            vst[vb][rr].load(vb_ + (int64_t)(it.key0 + key) * vss + dc * 8);
          else
            vst[vb][rr].zero();
        }
      }
    }
  };
  auto store = [&](unsigned char* Kb, unsigned char* Vb) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int ci = tid + c * NT;
      if (KCH % NT == 0 || ci < KCH) {
        const int row = ci / DC, col = ci % DC;
        *reinterpret_cast<uint4*>(Kb + row * KROW + col * 16) = kst[c].v;
      }
    }
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int bi = tid + vb * NT;
      if (VBL % NT == 0 || bi < VBL) {
        const int kg = bi / DC, dc = bi % DC;
        const uint4 r0 = vst[vb][0].v, r1 = vst[vb][1].v, r2 = vst[vb][2].v, r3 = vst[vb][3].v;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const uint32_t x0 = word(r0, dd >> 1), x1 = word(r1, dd >> 1);
          const uint32_t x2 = word(r2, dd >> 1), x3 = word(r3, dd >> 1);
          uint2 out;
          if ((dd & 1) == 0) {
            out.x = (x0 & 0xffffu) | (x1 << 16);
            out.y = (x2 & 0xffffu) | (x3 << 16);
          } else {
            out.x = (x0 >> 16) | (x1 & 0xffff0000u);
            out.y = (x2 >> 16) | (x3 & 0xffff0000u);
          }
          *reinterpret_cast<uint2*>(Vb + (dc * 8 + dd) * VROW + kg * 8) = out;
        }
      }
    }
  };

  const int arow = swap_b23(l32);
  // element mask of mask-list sub-tiles (causal or local): this row's kept keys
  const bool list_masked = p.mask_mod == kMaskCausal || p.mask_mod == kMaskLocal;
  int mlo, mhi;
  row_key_range(p.mask_mod, p.win_left, p.win_right, qrow, mlo, mhi);
  auto compute = [&](const unsigned char* Kb, const unsigned char* Vb, const Item& it) {
    f32x16_t s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(Kb + arow * KROW + ks * 32 + h32 * 16);
      const uint4 a1 =
          *reinterpret_cast<const uint4*>(Kb + (arow + 32) * KROW + ks * 32 + h32 * 16);
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
    }
    uint32_t pk0[8], pk1[8];
    if constexpr (PROXY) {
      softmax_step_any<DB>(s0, s1, it, xbits, p.block_kv, ti.num_n, ti.Sk, h32, p.c, m_run,
                           l_run, lo_run, oacc, pk0, pk1);
    } else {
      softmax_step<DB, true>(s0, s1, it, it.is_mask && list_masked, mlo, mhi, h32, p.c, m_run,
                             l_run, lo_run, oacc, pk0, pk1);
    }
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const uint4 bop = p_operand(pk0, pk1, ps);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint4 a =
            *reinterpret_cast<const uint4*>(Vb + (db * 32 + arow) * VROW + ps * 32 + h32 * 16);
        oacc[db] = mfma32(a, bop, oacc[db]);
      }
    }
  };

  ListWalk L{ti.mrow, p.mi_s[3], ti.mcnt, ti.frow, p.fi_s[3], ti.mcnt + ti.fcnt,
             p.block_kv, ti.num_n, p.mask_mod, ti.kvv, -1000000, -1, 0};
  unsigned char* buf0 = smem;
  unsigned char* buf1 = smem + STAGE;
  // listed blocks first, then (PROXY) the chunks of summaries with an unlisted block
  bool in_proxy = false;
  int pn = 0;
  auto step = [&](Item& it) -> bool {
    if (!in_proxy) {
      if (advance(it, L, lane, ti.Sk)) return true;
      in_proxy = true;
    }
    if constexpr (PROXY) return next_proxy_chunk(xbits, ti.num_n, pn, it);
    return false;
  };
  Item cur{-1, 0, 0, 0, 0, 0, 0};
  bool have = step(cur);
  if (have) {
    issue(cur);
    store(buf0, buf0 + KBYTES);
  }
  __syncthreads();
  Item nxt = cur;
  bool have_nxt = have && step(nxt);
  int sb = 0;
  while (have) {
    if (have_nxt) issue(nxt);
    unsigned char* cb = sb ? buf1 : buf0;
    unsigned char* ob = sb ? buf0 : buf1;
    if (live) compute(cb, cb + KBYTES, cur);
    if (have_nxt) store(ob, ob + KBYTES);
    __syncthreads();
    cur = nxt;
    have = have_nxt;
    if (have) have_nxt = step(nxt);
    sb ^= 1;
  }
  epilogue<DB, T>(p, ti, qrow, h32, m_run, l_run, lo_run, oacc);
}

template <int D, int NW, bool F32, bool PROXY>
hipError_t launch_one(const FwdParams& p, hipStream_t s) {
  FwdParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel(
      reinterpret_cast<const void*>(&bsa_fwd_staged_kernel<D, NW, F32, PROXY>),
      dim3(p.num_tiles), dim3(NW * 64), args, 0, s);
}

template <int D, bool F32, bool PROXY>
hipError_t launch_tm(const FwdParams& p, int tile_m, hipStream_t s) {
  switch (tile_m) {
    case 128: return launch_one<D, 4, F32, PROXY>(p, s);
    case 64: return launch_one<D, 2, F32, PROXY>(p, s);
    case 32: return launch_one<D, 1, F32, PROXY>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool F32, bool PROXY>
hipError_t launch_d(const FwdParams& p, int D, int tile_m, hipStream_t s) {
  switch (D) {
    case 64: return launch_tm<64, F32, PROXY>(p, tile_m, s);
    case 96: return launch_tm<96, F32, PROXY>(p, tile_m, s);
    case 128: return launch_tm<128, F32, PROXY>(p, tile_m, s);
    case 192: return launch_tm<192, F32, PROXY>(p, tile_m, s);
    case 256: return launch_tm<256, F32, PROXY>(p, tile_m, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_staged(const FwdParams& p, int D, int tile_m, bool f32_in, hipStream_t s) {
  return f32_in ? launch_d<true, false>(p, D, tile_m, s) : launch_d<false, false>(p, D, tile_m, s);
}

hipError_t launch_fwd_proxy_staged(const FwdParams& p, int D, int tile_m, hipStream_t s) {
  return launch_d<false, true>(p, D, tile_m, s);
}

}  // namespace bsa
