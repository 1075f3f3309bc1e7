// Block-sparse attention forward for gfx950 (CDNA4), bf16 Q/K/V.
//
// One workgroup owns TM = 32*NW query rows of one (batch, head) and walks
// only the KV blocks named by its rows' block lists (mask list first, then
// the full list), as the block-sparse forward of flash-attention PR #2224
// ("[CuTe,Flex] varlen blocksparsity") and the runtime-indexed K/V fetch of
// "Dense FlashAttention vs Block-Sparse Attention" (sections 4 and 6)
// describe: the address of the next tile comes from the block-index list,
// skipped blocks are never touched, and both K and V follow the index.
//
// Each listed KV block is cut into 64-key sub-tiles.  K and V rows go
// straight from HBM into LDS with 16-byte global_load_lds DMA (no staging
// registers), two stages, issued one sub-tile ahead: while sub-tile i
// computes from one stage, sub-tile i+1 streams into the other.  The DMA is
// issued from inline assembly so the compiler does not conservatively wait
// for it before every LDS read of the other stage; the kernel orders it
// itself: each sub-tile starts with vmcnt(0) (this wave's DMA landed) and a
// workgroup barrier (every wave's DMA landed, every wave finished reading
// the stage the next DMA overwrites).
//
// LDS layout: both tiles are [64 keys][RS 16-byte slots] with head-dim
// chunk c of key r at slot r*RS + c; the RS - D/8 slots at the end of a row
// are padding the DMA skips.  K is read as the S^T MFMA A operand with
// ds_read_b128: the 16 lanes of a quarter-wave read 16 different keys of one
// chunk, and an odd K stride puts them on 16 different bank groups.  V stays
// key-major and is read with ds_read_b64_tr_b16, which transposes 4x4 blocks
// of b16 inside each group of 16 lanes: source lane s of a group loads 4
// consecutive head dims of key kb + s/4, and lane i receives head dim d(i)
// of keys kb..kb+3, exactly the O^T MFMA A-operand layout.  Half a wave then
// reads 4 keys x 4 chunks, and a V stride of 4 or 12 (mod 16) slots puts
// those on 16 different bank groups.  Every read address is a per-lane base
// plus a compile-time offset.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_fwd_common.h"

namespace bsa {
namespace {

using namespace dev;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

// One wave-wide 16-byte-per-lane DMA: lane l's 16 bytes at base + off land
// at LDS byte address lds_addr + 16*l.  base (64-bit) and lds_addr must be
// wave-uniform: base goes in SGPRs (global "saddr" form, so a precomputed
// 32-bit lane offset is all the address arithmetic a lane needs), lds_addr
// in M0 (the s_nop covers the M0-write hazard).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "{m0}"(lds_addr)
               : "memory");
}

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt left alone): at most N of this wave's
// vector-memory ops, DMA included, still in flight.  Ops complete in order.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint2 read_tr(const uint4* lds, int byte_off) {
  lds_char* base = (lds_char*)(lds);  // generic -> LDS address space
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + byte_off));
  return __builtin_bit_cast(uint2, v);
}

template <int D, int NW>
struct FwdCfg {
  static constexpr int TM = NW * 32;
  static constexpr int DS = D / 16;  // QK^T k-steps
  static constexpr int DB = D / 32;  // O^T row blocks
  static constexpr int DC = D / 8;   // 16-byte chunks per row
  static constexpr int RSK = DC + 1;                                    // odd
  static constexpr int RSV = (DC % 16 == 4 || DC % 16 == 12) ? DC : DC + 4;  // 4 or 12 mod 16
  static constexpr int KSLOTS = kKvTile * RSK;  // = 64 * RSK: RSK DMA blocks of 64 slots
  static constexpr int VSLOTS = kKvTile * RSV;
  static constexpr int STAGE_SLOTS = KSLOTS + VSLOTS;  // K tile, then V tile
  static constexpr int STAGE_BYTES = STAGE_SLOTS * 16;
  // Up to 4 waves: two stages, so two workgroups share a CU.  8 waves (one
  // workgroup per CU, two waves per SIMD): three stages when they fit.
  static constexpr int STAGES = (NW == 8 && 3 * STAGE_BYTES <= 160 * 1024) ? 3 : 2;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int WAVES_PER_EU =
      NW == 8 ? 2 : (LDS_BYTES <= 80 * 1024 ? 2 : 1);
  static constexpr int KIPW = (RSK + NW - 1) / NW;  // K DMA instructions per wave per sub-tile
  static constexpr int VIPW = (RSV + NW - 1) / NW;
  static constexpr int DMA_PER_ITEM = KIPW + VIPW;
  static_assert(STAGES == 2 || DMA_PER_ITEM < 64, "vmcnt range");
  static_assert(DC % 2 == 0 && RSV % 16 != 0 && RSV % 4 == 0, "stride rules");
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(FwdCfg<D, NW>::WAVES_PER_EU)))
void bsa_fwd_kernel(const FwdParams p) {
  using C = FwdCfg<D, NW>;
  constexpr int DS = C::DS, DB = C::DB, DC = C::DC, RSK = C::RSK, RSV = C::RSV;
  __shared__ uint4 smem[C::STAGES * C::STAGE_SLOTS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, h32 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar

  TileInfo ti;
  if (!decode_tile<C::TM>(p, xcd_remap(blockIdx.x, p.num_tiles), ti)) return;
  const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + ti.qoff;
  const __bf16* kp = reinterpret_cast<const __bf16*>(p.k) + ti.koff;
  const __bf16* vp = reinterpret_cast<const __bf16*>(p.v) + ti.voff;

  // Q fragments (S^T MFMA B operand): Q[qrow][16*ks + 8*h32 .. +7]
  const int qrow = ti.q0 + 32 * w + l32;
  uint4 qf[DS];
#pragma unroll
  for (int ks = 0; ks < DS; ++ks)
    qf[ks] = qrow < ti.Sq
                 ? *reinterpret_cast<const uint4*>(qp + (int64_t)qrow * p.q_ss + ks * 16 + h32 * 8)
                 : make_uint4(0, 0, 0, 0);
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = neg_inf(), l_run = 0.f;

  // DMA of one 64-key sub-tile.  The tile's RS blocks of 64 slots are
  // dealt round-robin to the waves, each wave issuing the same number of
  // instructions (a wave with nothing left re-issues the last block, which
  // writes the same bytes again).  Lane l of block blk fills slot
  // 64*blk + l, i.e. key slot / RS, chunk slot % RS (a padding slot gets a
  // copy of the row's last chunk, which is never read).  Keys past nk repeat
  // the last visible key (finite data, masked later).  Lane byte offsets
  // within the sub-tile fit in 32 bits (the host bounds the row stride).
  constexpr int KIPW = C::KIPW, VIPW = C::VIPW, STAGES = C::STAGES;
  const int kss2 = p.k_ss * 2, vss2 = p.v_ss * 2;
  // lane byte offsets within a full sub-tile, one per DMA instruction
  uint32_t koff[KIPW], voff[VIPW];
#pragma unroll
  for (int ii = 0; ii < KIPW; ++ii) {
    const int slot = min(ii * NW + w, RSK - 1) * 64 + lane;
    koff[ii] = (slot / RSK) * kss2 + min(slot % RSK, DC - 1) * 16;
  }
#pragma unroll
  for (int ii = 0; ii < VIPW; ++ii) {
    const int slot = min(ii * NW + w, RSV - 1) * 64 + lane;
    voff[ii] = (slot / RSV) * vss2 + min(slot % RSV, DC - 1) * 16;
  }
  const uint32_t lds_base = (uint32_t)(size_t)((lds_char*)smem);
  auto issue = [&](const Item& it, int stage) {
    const char* kt = reinterpret_cast<const char*>(kp + it.key0 * p.k_ss);
    const char* vt = reinterpret_cast<const char*>(vp + it.key0 * p.v_ss);
    const uint32_t kl = lds_base + stage * C::STAGE_SLOTS * 16;
    const uint32_t vl = kl + C::KSLOTS * 16;
    if (it.nk == kKvTile) {
#pragma unroll
      for (int ii = 0; ii < KIPW; ++ii) dma16(kt, koff[ii], kl + min(ii * NW + w, RSK - 1) * 1024);
#pragma unroll
      for (int ii = 0; ii < VIPW; ++ii) dma16(vt, voff[ii], vl + min(ii * NW + w, RSV - 1) * 1024);
    } else {
      // partial sub-tile: keys past nk repeat the last visible key
      const int last = it.nk - 1;
#pragma unroll
      for (int ii = 0; ii < KIPW; ++ii) {
        const int blk = min(ii * NW + w, RSK - 1);
        const int slot = blk * 64 + lane;
        const int r = slot / RSK, c = min(slot % RSK, DC - 1);
        dma16(kt, min(r, last) * kss2 + c * 16, kl + blk * 1024);
      }
#pragma unroll
      for (int ii = 0; ii < VIPW; ++ii) {
        const int blk = min(ii * NW + w, RSV - 1);
        const int slot = blk * 64 + lane;
        const int r = slot / RSV, c = min(slot % RSV, DC - 1);
        dma16(vt, min(r, last) * vss2 + c * 16, vl + blk * 1024);
      }
    }
  };

  // per-lane read geometry
  const int arow = swap_b23(l32);
  const int kbase = (arow * RSK + h32) * 16;  // + kb*32*RSK*16 + ks*32 bytes
  const int vs = lane & 15, vg = lane >> 4;
  const int vkey = 8 * h32 + (vs >> 2);       // + 16*ps + 4*t
  const int vd = 16 * (vg & 1) + 4 * (((vs & 1) << 1) | ((vs >> 1) & 1));  // + 32*db
  const int vbase = (vkey * RSV + (vd >> 3)) * 16 + 8 * ((vd >> 2) & 1);

  auto compute = [&](int stage, const Item& it) {
    const uint4* kl = smem + stage * C::STAGE_SLOTS;
    const uint4* vl = kl + C::KSLOTS;
    f32x16_t s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
    const char* kb = reinterpret_cast<const char*>(kl) + kbase;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(kb + ks * 32);
      const uint4 a1 = *reinterpret_cast<const uint4*>(kb + 32 * RSK * 16 + ks * 32);
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
    }
    uint32_t pk0[8], pk1[8];
    softmax_step<DB>(s0, s1, it, it.is_mask && p.mask_mod == kMaskCausal, qrow, h32, p.c, m_run,
                     l_run, oacc, pk0, pk1);
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const uint4 bop = p_operand(pk0, pk1, ps);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = vbase + (16 * ps * RSV + 4 * db) * 16;
        const uint2 t0 = read_tr(vl, off);
        const uint2 t1 = read_tr(vl, off + 4 * RSV * 16);
        oacc[db] = mfma32(make_uint4(t0.x, t0.y, t1.x, t1.y), bop, oacc[db]);
      }
    }
  };

  ListWalk L{ti.mrow, p.mi_s[3], ti.mcnt, ti.frow, p.fi_s[3], ti.mcnt + ti.fcnt,
             p.block_kv, ti.num_n, p.mask_mod, p.kv_valid, -1000000, -1, 0};
  // STAGES-deep pipeline: up to STAGES-1 sub-tiles in flight ahead of the
  // one being computed.  The npend issued, not yet computed sub-tiles (p0
  // oldest, then p1) occupy stages stage, stage+1 (mod STAGES).
  Item walker{-1, 0, 0, 0, 0, 0, 0};
  bool more = advance(walker, L, lane, ti.Sk);
  Item p0 = walker, p1 = walker;
  int npend = 0;
  if (more) {
    issue(walker, 0);
    p0 = walker;
    npend = 1;
    more = advance(walker, L, lane, ti.Sk);
  }
  if constexpr (STAGES == 3) {
    if (more) {
      issue(walker, 1);
      p1 = walker;
      npend = 2;
      more = advance(walker, L, lane, ti.Sk);
    }
  }
  int stage = 0;
  while (npend > 0) {
    // the oldest pending sub-tile landed (for this wave), then for all waves;
    // every wave is also done computing the stage the next DMA overwrites
    if constexpr (STAGES == 3) {
      if (npend == 2)
        wait_vmem<C::DMA_PER_ITEM>();
      else
        wait_vmem<0>();
    } else {
      wait_vmem<0>();
    }
    __syncthreads();
    const Item cur = p0;
    if constexpr (STAGES == 3) p0 = p1;
    if (more) {
      int ns = stage + npend;
      if (ns >= STAGES) ns -= STAGES;
      issue(walker, ns);
      if (STAGES == 3 && npend == 2)
        p1 = walker;
      else
        p0 = walker;
      more = advance(walker, L, lane, ti.Sk);
    } else {
      --npend;
    }
    compute(stage, cur);
    stage = stage + 1 == STAGES ? 0 : stage + 1;
  }
  epilogue<DB, __bf16>(p, ti, qrow, h32, m_run, l_run, oacc);
}

template <int D, int NW>
hipError_t launch_one(const FwdParams& p, hipStream_t s) {
  FwdParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW>),
                         dim3(p.num_tiles), dim3(NW * 64), args, 0, s);
}

template <int D>
hipError_t launch_tm(const FwdParams& p, int tile_m, hipStream_t s) {
  switch (tile_m) {
    case 256:
      if constexpr (D <= 128) return launch_one<D, 8>(p, s);
      return hipErrorInvalidValue;
    case 128: return launch_one<D, 4>(p, s);
    case 64: return launch_one<D, 2>(p, s);
    case 32: return launch_one<D, 1>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int D, int tile_m, bool f32_in, hipStream_t s) {
  if (f32_in) return launch_fwd_staged(p, D, tile_m, true, s);
  if (tile_m == 256) return launch_fwd_pp(p, D, s);
  switch (D) {
    case 64: return launch_tm<64>(p, tile_m, s);
    case 96: return launch_tm<96>(p, tile_m, s);
    case 128: return launch_tm<128>(p, tile_m, s);
    case 192: return launch_tm<192>(p, tile_m, s);
    case 256: return launch_tm<256>(p, tile_m, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bsa
