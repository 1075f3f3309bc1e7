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
// registers).  With two stages, sub-tile i+1 streams into one stage while
// sub-tile i computes from the other.  With one stage (chosen where the
// smaller LDS footprint lets more workgroups share a CU), sub-tile i+1 is
// fetched once every wave has finished with sub-tile i, and the other
// workgroups on the CU compute meanwhile.  The DMA is issued from inline
// assembly so the compiler does not conservatively wait for it before every
// LDS read; the kernel orders it itself: each sub-tile starts with vmcnt(0)
// (this wave's DMA landed) and a workgroup barrier (every wave's DMA landed,
// every wave finished reading the stage the next DMA overwrites).
//
// LDS layout: both tiles are [64 keys][RS 16-byte slots].  K is read as the
// S^T MFMA A operand with ds_read_b128: the 16 lanes of a quarter-wave read
// one chunk of 16 different keys.  V stays key-major and is read with
// ds_read_b64_tr_b16, which transposes 4x4 blocks of b16 inside each group
// of 16 lanes: source lane s of a group loads 4 consecutive head dims of key
// kb + s/4, and lane i receives head dim d(i) of keys kb..kb+3, exactly the
// O^T MFMA A-operand layout; half a wave then reads 4 keys x 4 chunks.  For
// head_dim 64, 128 and 256 rows are unpadded (RS = D/8) and chunk c of key r
// sits at position c ^ swz(r): K uses swz = r & 15 (D >= 128) or
// (r >> 1) & 7 (D = 64), which puts the 16 keys of a quarter-wave on 16
// different 16-byte bank groups; V uses swz = 4 * (r & 3) (D >= 128) or
// 4 * ((r >> 1) & 1) (D = 64), which puts the 4 keys of a half-wave on the 4
// quarters of the banks.  The k-step and the head-dim block enter the read
// address as an XOR on bits 4..8, so a lane keeps one address per K k-step
// and per V head-dim block.  Head_dim 96 and 192 pad instead: chunk c at
// slot r*RS + c, an odd K stride and a V stride of 4 or 12 (mod 16) slots;
// every read address is then a per-lane base plus a compile-time offset.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_fwd_common.h"
#include "bsa_fwd_proxy.h"

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
// in M0.  The compiler's hazard checks do not see inside the asm, so its
// s_nop 4 provides the wait states the load needs after the instructions
// that set its operands: one after the M0 write, and five after a VALU
// instruction that writes an SGPR a vector-memory instruction reads (the
// base is often restored from a spill with v_readlane just before; with
// fewer wait states the load can take a stale base and fault).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
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
  // D = 64, 128, 256: unpadded rows, chunk c of key r at position c ^ swz(r)
  // (the swizzle of the 256-row kernel; D = 256 rows hold 32 chunks and the
  // same K and V swizzles keep both read patterns free of bank conflicts).
  // D = 96, 192: padded rows, odd K stride, V stride 4 or 12 (mod 16).
  static constexpr bool SWZ = D == 64 || D == 128 || D == 256;
  static constexpr int RSK = SWZ ? DC : DC + 1;
  static constexpr int RSV = SWZ ? DC : (DC % 16 == 4 || DC % 16 == 12) ? DC : DC + 4;
  static constexpr int KSLOTS = kKvTile * RSK;  // = 64 * RSK: RSK DMA blocks of 64 slots
  static constexpr int VSLOTS = kKvTile * RSV;
  static constexpr int STAGE_SLOTS = KSLOTS + VSLOTS;  // K tile, then V tile
  static constexpr int STAGE_BYTES = STAGE_SLOTS * 16;
  // One stage (the next sub-tile is fetched once the current one is done)
  // or two (it streams in while the current one computes), chosen by
  // measurement on the 25 %-density sweep (TFLOP/s, two stages -> one):
  //   128-row tiles: one at d = 128 (664 -> 694) and d = 192 (481 -> 552,
  //     two workgroups per CU instead of one); two at d = 64 (-2 % with one)
  //     and d = 256 (-11 %)
  //   64-row tiles: one (d = 128, (64,128): 400 -> 542, four workgroups per
  //     CU hide each other's fetch and softmax; d = 192: 273 -> 436-481 and
  //     d = 256: 201 -> 411, two workgroups per CU instead of one)
  //   32-row tiles: one at d <= 128, two above
  static constexpr int stages() {
    if (NW == 4) return (D == 128 || D == 192) ? 1 : 2;
    if (NW == 2) return 1;
    return D <= 128 ? 1 : 2;
  }
  static constexpr int STAGES = stages();
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // Register budget: 256 per wave (two waves per SIMD) when the LDS lets
  // eight or more waves share a CU, else 512.  A 64-row tile at d = 192 or
  // 256 fits two workgroups (four waves) per CU: one wave per SIMD, so the
  // larger budget costs no occupancy and removes the spills.
  static constexpr int WGS_PER_CU_BY_LDS = (160 * 1024) / LDS_BYTES;
  static constexpr int WAVES_PER_EU =
      NW == 1 ? (LDS_BYTES <= 80 * 1024 ? 2 : 1) : (WGS_PER_CU_BY_LDS * NW >= 8 ? 2 : 1);
  static constexpr int KIPW = (RSK + NW - 1) / NW;  // most K DMA instructions of a wave per sub-tile
  static constexpr int VIPW = (RSV + NW - 1) / NW;
  // Swizzled rows: DMA block ii of a wave covers keys (ii*NW + w) * 64/RS ..,
  // so its lane offsets repeat every KP (VP) blocks up to a wave-uniform key
  // step (the K swizzle has a period of 16 keys, the V swizzle of 4), and
  // only KP (VP) offsets per lane are kept.  Padded rows keep one per block.
  static constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }
  static constexpr int KSTEP = SWZ ? NW * 64 / RSK : 0;  // keys between blocks ii and ii+1
  static constexpr int VSTEP = SWZ ? NW * 64 / RSV : 0;
  static constexpr int KP = SWZ ? 16 / gcd(16, KSTEP) : KIPW;
  static constexpr int VP = SWZ ? 4 / gcd(4, VSTEP) : VIPW;
  static_assert(NW <= 4, "256-row tiles run in the ping-pong kernel");
  static_assert(DC % 2 == 0 && (SWZ || (RSK % 2 == 1 && RSV % 16 != 0 && RSV % 4 == 0)),
                "stride rules");
  __device__ __forceinline__ static int kswz(int r) {
    return D >= 128 ? (r & 15) : D == 64 ? ((r >> 1) & 7) : 0;
  }
  __device__ __forceinline__ static int vswz(int r) {
    return D >= 128 ? 4 * (r & 3) : D == 64 ? 4 * ((r >> 1) & 1) : 0;
  }
};

// LOCAL: the local mask_mod's key range on mask-list sub-tiles (a separate
// instance, so the others keep the plain causal test).
// PACK: items are packed from the keys of consecutive listed blocks
// (advance_packed), K/V rows gathered per lane from up to kPackSeg runs.
template <int D, int NW, bool LOCAL, bool PROXY, bool VARLEN, bool PACK>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(FwdCfg<D, NW>::WAVES_PER_EU)))
void bsa_fwd_kernel(const FwdParams p) {
  using C = FwdCfg<D, NW>;
  constexpr int DS = C::DS, DB = C::DB, DC = C::DC, RSK = C::RSK, RSV = C::RSV;
  __shared__ uint4 smem[C::STAGES * C::STAGE_SLOTS];
  __shared__ uint32_t xbits[PROXY ? kProxyBitmapWords : 1];  // listed blocks (proxy route)

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, h32 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar

  TileInfo ti;
  const int tix = xcd_remap(blockIdx.x, p.num_tiles);
  if (!decode_tile<C::TM, VARLEN ? 1 : 0>(p, tix, ti)) return;
  const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + ti.qoff;
  const __bf16* kp = reinterpret_cast<const __bf16*>(p.k) + ti.koff;
  const __bf16* vp = reinterpret_cast<const __bf16*>(p.v) + ti.voff;
  // proxy route (batched; summaries share K's and V's row strides, so the DMA
  // lane offsets below serve both)
  const __bf16* ksp = nullptr;
  const __bf16* vsp = nullptr;
  if constexpr (PROXY) {
    const int bh = tix / p.tiles_per_head;
    const int b = bh / p.H, hk = (bh % p.H) / p.hrep;
    ksp = reinterpret_cast<const __bf16*>(p.ksum) + b * p.ks_sb + hk * p.ks_sh;
    vsp = reinterpret_cast<const __bf16*>(p.vsum) + b * p.vs_sb + hk * p.vs_sh;
    build_listed_bitmap(xbits, p, ti, tid, NW * 64);
  }

  // Q fragments (S^T MFMA B operand): Q[qrow][16*ks + 8*h32 .. +7].  A wave
  // whose 32 rows all lie past the Q block's end (a block that is not a
  // multiple of 32 rows) only fetches and waits with the others.
  const int qrow = ti.q0 + 32 * w + l32;
  const bool live = ti.q0 + 32 * w < ti.qend;
  // The first 64 list entries are fetched before Q: the first K/V DMA waits
  // only for them, while Q is still in flight (vector loads complete in
  // order, so a wait for a list entry fetched after Q would wait for Q too).
  ListWalk L{ti.mrow, p.mi_s[3], ti.mcnt, ti.frow, p.fi_s[3], ti.mcnt + ti.fcnt,
             p.block_kv, ti.num_n, p.mask_mod, ti.kvv, -1000000, -1, 0};
  L.fetch(0, lane);
  uint4 qf[DS];
#pragma unroll
  for (int ks = 0; ks < DS; ++ks)
    qf[ks] = qrow < ti.qend
                 ? *reinterpret_cast<const uint4*>(qp + (int64_t)qrow * p.q_ss + ks * 16 + h32 * 8)
                 : make_uint4(0, 0, 0, 0);
  L.lengths(lane);
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = neg_inf(), l_run = 0.f, lo_run = 0.f;

  // DMA of one 64-key sub-tile.  The tile's RS blocks of 64 slots are
  // dealt round-robin to the waves; a wave issues only the blocks that
  // exist (each sub-tile ends with vmcnt(0), so the counts need not match).
  // Lane l of block blk fills slot 64*blk + l, i.e. key slot / RS at chunk
  // position slot % RS, which holds chunk position ^ swz(key) (swizzled
  // rows) or the chunk itself (padded rows: a padding slot gets a copy of
  // the row's last chunk, never read).  Keys past nk repeat the last visible
  // key (finite data, masked later).  Lane byte offsets within the sub-tile
  // fit in 32 bits (the host bounds the row stride).
  constexpr int KIPW = C::KIPW, VIPW = C::VIPW, STAGES = C::STAGES;
  const int kss2 = p.k_ss * 2, vss2 = p.v_ss * 2;
  // source chunk stored at chunk position pos of key row `key` (K or V tile)
  auto kchunk = [&](int key, int pos) { return C::SWZ ? pos ^ C::kswz(key) : min(pos, DC - 1); };
  auto vchunk = [&](int key, int pos) { return C::SWZ ? pos ^ C::vswz(key) : min(pos, DC - 1); };
  // lane byte offsets within a full sub-tile for the first KP (VP) DMA
  // blocks of this wave; block ii uses entry ii % KP and a key step
  // Padded rows with many DMA blocks under the 256-register budget (d = 192,
  // 128-row tiles) compute the offsets when they issue (a few VALU per DMA)
  // rather than keep one register per block, which spilled.
  constexpr bool OTF = !C::SWZ && C::WAVES_PER_EU == 2 && D >= 192;
  constexpr int KP = OTF ? 1 : C::KP < KIPW ? C::KP : KIPW;
  constexpr int VP = OTF ? 1 : C::VP < VIPW ? C::VP : VIPW;
  auto kofs = [&](int ii) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // computed at the DMA, not hoisted into a live register
    const int slot = min(ii * NW + w, RSK - 1) * 64 + ln;
    return (uint32_t)((slot / RSK) * kss2 + kchunk(slot / RSK, slot % RSK) * 16);
  };
  auto vofs = [&](int ii) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int slot = min(ii * NW + w, RSV - 1) * 64 + ln;
    return (uint32_t)((slot / RSV) * vss2 + vchunk(slot / RSV, slot % RSV) * 16);
  };
  uint32_t koff[KP], voff[VP];
#pragma unroll
  for (int ii = 0; ii < KP; ++ii) {
    const int slot = min(ii * NW + w, RSK - 1) * 64 + lane;
    koff[ii] = (slot / RSK) * kss2 + kchunk(slot / RSK, slot % RSK) * 16;
  }
#pragma unroll
  for (int ii = 0; ii < VP; ++ii) {
    const int slot = min(ii * NW + w, RSV - 1) * 64 + lane;
    voff[ii] = (slot / RSV) * vss2 + vchunk(slot / RSV, slot % RSV) * 16;
  }
  const uint32_t lds_base = (uint32_t)(size_t)((lds_char*)smem);
  auto issue = [&](const Item& it, int stage) {
    // the item is wave-uniform; the proxy instance says so explicitly, since
    // the chunk walk's LDS reads hide it from the compiler (DMA bases are SGPRs)
    const bool px = PROXY && __builtin_amdgcn_readfirstlane(it.is_mask) == 2;
    const int key0 = PROXY ? __builtin_amdgcn_readfirstlane(it.key0) : it.key0;
    const char* kt = reinterpret_cast<const char*>((px ? ksp : kp) + key0 * p.k_ss);
    const char* vt = reinterpret_cast<const char*>((px ? vsp : vp) + key0 * p.v_ss);
    const uint32_t kl = lds_base + stage * C::STAGE_SLOTS * 16;
    const uint32_t vl = kl + C::KSLOTS * 16;
    // block ii*NW + w exists unless it is the last one of a wave and past RS
    auto kblk = [&](int ii) { return !(RSK % NW != 0 && ii == KIPW - 1 && ii * NW + w >= RSK); };
    auto vblk = [&](int ii) { return !(RSV % NW != 0 && ii == VIPW - 1 && ii * NW + w >= RSV); };
    if constexpr (PACK) {
      // gathered item: row r of the tile holds sequence key r + d_s of the run
      // s it falls in (rows past nk repeat the last key); byte offsets from
      // the sequence's first K/V row fit in 31 bits (checked by the host)
      const int last = it.nk - 1;
      // wave-uniform run bounds and offsets as plain values (selects between
      // struct fields would become an indexed load from scratch)
      const int e0 = __builtin_amdgcn_readfirstlane(it.e0);
      const int e1 = __builtin_amdgcn_readfirstlane(it.e1);
      const int e2 = __builtin_amdgcn_readfirstlane(it.e2);
      const int d0 = __builtin_amdgcn_readfirstlane(it.d0);
      const int d1 = __builtin_amdgcn_readfirstlane(it.d1);
      const int d2 = __builtin_amdgcn_readfirstlane(it.d2);
      const int d3 = __builtin_amdgcn_readfirstlane(it.d3);
      // sum of steps rather than a select chain, which the compiler would
      // turn into a lookup table in scratch memory
      const int q1 = d1 - d0, q2 = d2 - d1, q3 = d3 - d2;
      auto gkey = [=](int r) {
        const int rr = min(r, last);
        return rr + d0 + q1 * (int)(rr >= e0) + q2 * (int)(rr >= e1) + q3 * (int)(rr >= e2);
      };
      const char* kb = reinterpret_cast<const char*>(kp);
      const char* vb = reinterpret_cast<const char*>(vp);
#pragma unroll
      for (int ii = 0; ii < KIPW; ++ii) {
        if (!kblk(ii)) continue;
        const int slot = (ii * NW + w) * 64 + lane;
        const int r = slot / RSK;
        dma16(kb, (uint32_t)(gkey(r) * kss2 + kchunk(r, slot % RSK) * 16),
              kl + (ii * NW + w) * 1024);
      }
#pragma unroll
      for (int ii = 0; ii < VIPW; ++ii) {
        if (!vblk(ii)) continue;
        const int slot = (ii * NW + w) * 64 + lane;
        const int r = slot / RSV;
        dma16(vb, (uint32_t)(gkey(r) * vss2 + vchunk(r, slot % RSV) * 16),
              vl + (ii * NW + w) * 1024);
      }
    } else if (it.nk == kKvTile) {
#pragma unroll
      for (int ii = 0; ii < KIPW; ++ii)
        if (kblk(ii))
          dma16(kt + (ii / KP) * (KP * C::KSTEP) * kss2, OTF ? kofs(ii) : koff[ii % KP],
                kl + (ii * NW + w) * 1024);
#pragma unroll
      for (int ii = 0; ii < VIPW; ++ii)
        if (vblk(ii))
          dma16(vt + (ii / VP) * (VP * C::VSTEP) * vss2, OTF ? vofs(ii) : voff[ii % VP],
                vl + (ii * NW + w) * 1024);
    } else {
      // partial sub-tile: keys past nk repeat the last visible key (laid out
      // with the destination row's swizzle)
      const int last = it.nk - 1;
#pragma unroll
      for (int ii = 0; ii < KIPW; ++ii) {
        if (!kblk(ii)) continue;
        const int slot = (ii * NW + w) * 64 + lane;
        const int r = slot / RSK;
        dma16(kt, min(r, last) * kss2 + kchunk(r, slot % RSK) * 16, kl + (ii * NW + w) * 1024);
      }
#pragma unroll
      for (int ii = 0; ii < VIPW; ++ii) {
        if (!vblk(ii)) continue;
        const int slot = (ii * NW + w) * 64 + lane;
        const int r = slot / RSV;
        dma16(vt, min(r, last) * vss2 + vchunk(r, slot % RSV) * 16, vl + (ii * NW + w) * 1024);
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
  // swizzled rows: the k-step (K) and the head-dim block (V) enter as an XOR
  // on address bits 4..8; the key offsets added after it leave those alone
  int kx[C::SWZ ? DS : 1], vx[C::SWZ ? DB : 1];
  if constexpr (C::SWZ) {
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
      kx[ks] = (arow * RSK * 16 + 16 * (h32 ^ C::kswz(arow))) ^ (32 * ks);
#pragma unroll
    for (int db = 0; db < DB; ++db) vx[db] = (vbase + 16 * C::vswz(vkey)) ^ (64 * db);
  }

  // element mask of mask-list sub-tiles (causal or local): this row's kept keys
  const bool list_masked = LOCAL || p.mask_mod == kMaskCausal;
  int mlo = 0, mhi = qrow;
  if constexpr (LOCAL) row_key_range(kMaskLocal, p.win_left, p.win_right, qrow, mlo, mhi);
  auto compute = [&](int stage, const Item& it) {
    const uint4* kl = smem + stage * C::STAGE_SLOTS;
    const uint4* vl = kl + C::KSLOTS;
    f32x16_t s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
    // Both products read their LDS operands one step ahead of the MFMAs that
    // use them and no further (sched_barrier): left to itself the compiler
    // hoists every read of the loop, and the registers that takes spill at
    // d = 192 and cost occupancy elsewhere.
    const char* kb = reinterpret_cast<const char*>(kl) + (C::SWZ ? 0 : kbase);
    auto kld = [&](int ks, int half) {
      const int ko = C::SWZ ? kx[C::SWZ ? ks : 0] : ks * 32;
      return *reinterpret_cast<const uint4*>(kb + ko + half * 32 * RSK * 16);
    };
    uint4 n0 = kld(0, 0), n1 = kld(0, 1);
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const uint4 a0 = n0, a1 = n1;
      if (ks + 1 < DS) {
        n0 = kld(ks + 1, 0);
        n1 = kld(ks + 1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t pk0[8], pk1[8];
    if constexpr (PROXY)
      softmax_step_any<DB>(s0, s1, it, xbits, p.block_kv, ti.num_n, ti.Sk, h32, p.c, m_run,
                           l_run, lo_run, oacc, pk0, pk1);
    else
      softmax_step<DB, LOCAL, PACK>(s0, s1, it, it.is_mask != 0 && list_masked, mlo, mhi, h32,
                                    p.c, m_run, l_run, lo_run, oacc, pk0, pk1);
    // PV step i: keys 16*(i / DB) .., head dims 32*(i % DB) ..
    auto vld = [&](int i) {
      const int ps = i / DB, db = i % DB;
      const int off = C::SWZ ? vx[C::SWZ ? db : 0] + 16 * ps * RSV * 16
                             : vbase + (16 * ps * RSV + 4 * db) * 16;
      const uint2 t0 = read_tr(vl, off);
      const uint2 t1 = read_tr(vl, off + 4 * RSV * 16);
      return make_uint4(t0.x, t0.y, t1.x, t1.y);
    };
    uint4 nv = vld(0);
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      const uint4 a = nv;
      if (i + 1 < 4 * DB) nv = vld(i + 1);
      __builtin_amdgcn_sched_barrier(0);
      oacc[i % DB] = mfma32(a, p_operand(pk0, pk1, i / DB), oacc[i % DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Two stages: the sub-tile after the one being computed streams into the
  // other stage.  One stage: the next sub-tile is fetched once every wave is
  // done with the current one.  p0 is the issued, not yet computed sub-tile.
  // listed blocks, then (PROXY) the chunks of summaries holding an unlisted block
  bool in_proxy = false;
  int pn = 0;
  auto step = [&](Item& it) -> bool {
    if (!in_proxy) {
      if constexpr (PACK) return advance_packed(it, L, lane, ti.Sk, list_masked);
      if (advance(it, L, lane, ti.Sk)) return true;
      in_proxy = true;
    }
    if constexpr (PROXY) return next_proxy_chunk(xbits, ti.num_n, pn, it);
    return false;
  };
  Item walker{-1, 0, 0, 0, 0, 0, 0, kKvTile, kKvTile, kKvTile, 0, 0, 0, 0};
  bool more = step(walker);
  Item p0 = walker;
  bool pending = false;
  if (more) {
    issue(walker, 0);
    p0 = walker;
    pending = true;
    more = step(walker);
  }
  int stage = 0;
  if constexpr (STAGES == 1) {
    while (pending) {
      wait_vmem<0>();
      __syncthreads();
      const Item cur = p0;
      if (live) compute(0, cur);
      if (more) {
        __syncthreads();  // every wave done with the stage before it is refilled
        issue(walker, 0);
        p0 = walker;
        more = step(walker);
      } else {
        pending = false;
      }
    }
  }
  while (STAGES == 2 && pending) {
    // the pending sub-tile landed (for this wave), then for all waves; every
    // wave is also done computing the stage the next DMA overwrites
    wait_vmem<0>();
    __syncthreads();
    const Item cur = p0;
    if (more) {
      issue(walker, stage ^ 1);
      p0 = walker;
      more = step(walker);
    } else {
      pending = false;
    }
    if (live) compute(stage, cur);
    stage ^= 1;
  }
  epilogue<DB, __bf16>(p, ti, qrow, h32, m_run, l_run, lo_run, oacc);
}

// The packed-item instance (none for 32-row tiles at head_dim >= 192, whose
// registers would spill; the host does not pack those).
template <int D, int NW>
const void* pack_kernel() {
  if constexpr (NW == 1 && D >= 192)
    return reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW, false, false, false, false>);
  else
    return reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW, false, false, false, true>);
}

template <int D, int NW>
hipError_t launch_one(const FwdParams& p, hipStream_t s) {
  FwdParams copy = p;
  void* args[] = {&copy};
  // batched and packed-varlen tile decodes are separate instances; packed
  // items (route packing) are batched only
  const void* k =
      p.ksum ? reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW, false, true, false, false>)
      : p.mask_mod == kMaskLocal
          ? (p.varlen
                 ? reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW, true, false, true, false>)
                 : reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW, true, false, false, false>))
      : p.varlen ? reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW, false, false, true, false>)
      : p.pack   ? pack_kernel<D, NW>()
                 : reinterpret_cast<const void*>(&bsa_fwd_kernel<D, NW, false, false, false, false>);
  return hipLaunchKernel(k, dim3(p.num_tiles), dim3(NW * 64), args, 0, s);
}

template <int D>
hipError_t launch_tm(const FwdParams& p, int tile_m, hipStream_t s) {
  switch (tile_m) {  // 256-row tiles run in the ping-pong kernel
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
