// H += 2 X^T X on gfx950: bf16 MFMA with fp32 accumulation.
//
// "GPTQ" (wikiprompt.org), "Enfoque Técnico": the method works from the
// Hessian of the layer loss built from calibration inputs; for a linear
// layer that is (up to the factor 2 kept here) the Gram matrix of the
// calibration activations X (T tokens x n input channels).
//
// Design (MI355X):
//  * Only output tiles on or above the diagonal are computed (symmetry).
//  * 256x256 output tile per workgroup, accumulated by
//    v_mfma_f32_32x32x16_bf16.
//  * X is row-major (tokens x channels) while MFMA wants 8 consecutive
//    tokens of one channel per lane. For 16-byte aligned X the tile streams
//    through a 4-deep LDS ring filled by LDS-DMA in X's own layout and read
//    with gfx950's transposing LDS reads (k_hessian_dma below: 8 waves, each
//    a 128x64 block of 4x2 accumulators, 128 fp32 per lane). Other X (odd
//    row stride) takes k_hessian_bf16: 4 waves, each a 128x128 block (256
//    fp32 per lane, held in AGPRs), fed by 16-byte register loads of 8x8
//    blocks transposed with v_perm_b32 into a [channel][token] LDS layout.
//  * The token range is split into chunks; each chunk writes an fp32 partial
//    Gram matrix and a second kernel sums the partials in a fixed order,
//    scales by 2, adds to H and mirrors it: deterministic, exactly
//    symmetric, and the chunked sum bounds fp32 accumulation error. The
//    number of chunks is chosen so that tiles x chunks fills whole waves of
//    the 256 CUs (one 128-160 KiB workgroup per CU).
#include "common.h"
#include "dma.h"

#include <utility>

#include <type_traits>

namespace gq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kHT = 256;      // output tile edge
constexpr int kHBK = 64;      // tokens per LDS stage
constexpr int kHPitch = 36;   // dwords per LDS row (32 data + 4 pad)
constexpr int kHStage = kHT * kHPitch;  // dwords per operand per stage

int hessian_splits(int64_t T, int64_t n) {
  // Chunks of at least 4096 tokens (fp32 accumulation of a chunk stays
  // ~1e-6 relative) and at most 16; among the candidates the count whose
  // workgroups fill the 256 CUs best, the smallest on ties.
  const int64_t nt = ceil_div(n, 256);
  const int64_t tiles = nt * (nt + 1) / 2;
  int64_t lo = ceil_div(T, 65536), hi = ceil_div(T, 4096);
  if (lo < 1) lo = 1;
  if (hi > 16) hi = 16;
  if (lo > hi) lo = hi;
  int best = (int)lo;
  double best_fill = -1.0;
  for (int64_t sp = lo; sp <= hi; ++sp) {
    const int64_t items = tiles * sp;
    const double fill = (double)items / (double)(256 * ceil_div(items, 256));
    if (fill > best_fill + 1e-9) { best_fill = fill; best = (int)sp; }
  }
  return best;
}

__device__ inline void upper_tile(int t, int nt, int& bi, int& bj) {
  // enumerate (bi, bj), bi <= bj, row by row
  int row = 0;
  while (t >= nt - row) { t -= nt - row; ++row; }
  bi = row;
  bj = row + t;
}

// Work item of block b: (split, tile), from the split-major item list (tile
// fastest). The dispatcher deals consecutive block ids to the 8 XCDs in
// turn, and an XCD holds one of these 128 KiB workgroups per CU, 32 at a
// time. Blocks are read as rounds of 256: in round r, XCD x takes items
// 256 r + 32 x ... 256 r + 32 x + 31. The 32 workgroups resident on an XCD
// then work on consecutive tiles of one token chunk (their channel strips
// meet in that XCD's L2), and the whole chip stays within about two
// adjacent chunks at a time (144 MB of X at n = 4096), which the 256 MB
// last-level cache holds while the XCDs re-read it.
// Returns false for padding blocks (the grid is a whole number of rounds).
__device__ inline bool hessian_item(int b, int ntile, int splits, int& tile, int& split) {
  const int q = b >> 3;
  const int w = (((q >> 5) << 3) + (b & 7)) * 32 + (q & 31);
  if (w >= ntile * splits) return false;
  split = w / ntile;
  tile = w - split * ntile;
  return true;
}

// Load an 8(token) x 8(channel) bf16 block: rows X[t0+r][c0..c0+7].
template <bool kAligned>
__device__ inline void load_block(const uint16_t* __restrict__ X, int64_t ldx, int64_t t0,
                                  int64_t tend, int64_t c0, int64_t n, uint4 (&d)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    int64_t t = t0 + r;
    if (kAligned) {
      if (t < tend && c0 < n) {
        d[r] = *reinterpret_cast<const uint4*>(X + t * ldx + c0);
      } else {
        d[r] = make_uint4(0, 0, 0, 0);
      }
    } else {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t lo = 0, hi = 0;
        int64_t c = c0 + 2 * q;
        if (t < tend && c < n) lo = X[t * ldx + c];
        if (t < tend && c + 1 < n) hi = X[t * ldx + c + 1];
        w[q] = lo | (hi << 16);
      }
      d[r] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Transpose the block in registers and store channel rows into LDS.
__device__ inline void store_block_t(uint32_t* __restrict__ s, int row0, int tok_dw,
                                     const uint4 (&d)[8]) {
  uint32_t dd[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    dd[r][0] = d[r].x; dd[r][1] = d[r].y; dd[r][2] = d[r].z; dd[r][3] = d[r].w;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t ev[4], od[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // channel 2q is the low half of dword q, channel 2q+1 the high half;
      // pack tokens (2p, 2p+1) into one dword
      ev[p] = __builtin_amdgcn_perm(dd[2 * p + 1][q], dd[2 * p][q], 0x05040100u);
      od[p] = __builtin_amdgcn_perm(dd[2 * p + 1][q], dd[2 * p][q], 0x07060302u);
    }
    *reinterpret_cast<uint4*>(s + (row0 + 2 * q) * kHPitch + tok_dw) =
        make_uint4(ev[0], ev[1], ev[2], ev[3]);
    *reinterpret_cast<uint4*>(s + (row0 + 2 * q + 1) * kHPitch + tok_dw) =
        make_uint4(od[0], od[1], od[2], od[3]);
  }
}

template <bool kAligned>
__global__ void __launch_bounds__(256)
k_hessian_bf16(const uint16_t* __restrict__ X, int64_t T, int64_t n, int64_t ldx,
               float* __restrict__ part, int64_t chunk) {
  __shared__ uint32_t smem[2 * 2 * kHStage];
  const int nt = (int)ceil_div(n, kHT);
  int bi, bj;
  const int split = (int)blockIdx.x / (nt * (nt + 1) / 2);
  upper_tile((int)blockIdx.x - split * (nt * (nt + 1) / 2), nt, bi, bj);
  const int64_t kbeg = (int64_t)split * chunk;
  const int64_t kend = min(T, kbeg + chunk);
  const int64_t iA = (int64_t)bi * kHT, iB = (int64_t)bj * kHT;
  float* __restrict__ P = part + (int64_t)split * n * n;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // loader coordinates: 32 channel blocks x 8 token blocks
  const int lb_c = tid >> 3, lb_t = tid & 7;

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int64_t nstage = kend > kbeg ? ceil_div(kend - kbeg, kHBK) : 0;
  uint4 ra[8], rb[8];
  if (nstage > 0) {
    load_block<kAligned>(X, ldx, kbeg + 8 * lb_t, kend, iA + 8 * lb_c, n, ra);
    load_block<kAligned>(X, ldx, kbeg + 8 * lb_t, kend, iB + 8 * lb_c, n, rb);
    store_block_t(smem, 8 * lb_c, 4 * lb_t, ra);
    store_block_t(smem + kHStage, 8 * lb_c, 4 * lb_t, rb);
  }
  __syncthreads();

  for (int64_t st = 0; st < nstage; ++st) {
    const int cur = (int)(st & 1);
    const bool more = st + 1 < nstage;
    if (more) {
      const int64_t t0 = kbeg + (st + 1) * kHBK + 8 * lb_t;
      load_block<kAligned>(X, ldx, t0, kend, iA + 8 * lb_c, n, ra);
      load_block<kAligned>(X, ldx, t0, kend, iB + 8 * lb_c, n, rb);
    }
    const uint32_t* sA = smem + cur * 2 * kHStage;
    const uint32_t* sB = sA + kHStage;
#pragma unroll
    for (int ks = 0; ks < kHBK / 16; ++ks) {
      bf16x8_t af[4], bfr[4];
      const int koff = 8 * ks + 4 * (lane >> 5);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = 128 * wm + 32 * mb + (lane & 31);
        uint4 v = *reinterpret_cast<const uint4*>(sA + row * kHPitch + koff);
        af[mb] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int row = 128 * wn + 32 * nb + (lane & 31);
        uint4 v = *reinterpret_cast<const uint4*>(sB + row * kHPitch + koff);
        bfr[nb] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) {
      uint32_t* dA = smem + (cur ^ 1) * 2 * kHStage;
      store_block_t(dA, 8 * lb_c, 4 * lb_t, ra);
      store_block_t(dA + kHStage, 8 * lb_c, 4 * lb_t, rb);
    }
    __syncthreads();
  }

  // epilogue: lane holds D[i][j], j = lane%32, i = 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = iA + 128 * wm + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t j = iB + 128 * wn + 32 * nb + (lane & 31);
        if (i < n && j < n) P[i * n + j] = acc[mb][nb][r];
      }
}

// ---------------------------------------------------------------------------
// Streaming variant for 16-byte aligned X: buffer LDS-DMA staging and
// transposing LDS reads.
//
//  * buffer_load_dwordx4 ... lds moves 16-byte chunks (8 channels of one
//    token) straight from HBM into LDS without passing through VGPRs, so a
//    ring of four 32-token stages (128 KiB of LDS) keeps the fill two
//    stages ahead of the one being multiplied. The buffer
//    descriptor spans this workgroup's token chunk, so each lane's offset is
//    fixed and one scalar offset advances a whole stage; chunks past the
//    chunk's last token or the last channel are outside the descriptor's
//    range and read as zeros (the hardware bounds check), so the loop has
//    no per-chunk predication.
//  * LDS keeps X's own layout, [token][channel] with 512-byte rows per
//    operand; the 16-byte chunk index of row t is XOR-swizzled with
//    dma_swz(t) (each DMA lane fetches the global chunk that belongs to its
//    fixed LDS slot).
//  * ds_read_b64_tr_b16 turns it into MFMA operands (4 consecutive tokens of
//    one channel per read, two reads per 8-token K slice). A group's 16
//    reads hit 4 rows x 32 bytes; the swizzle spreads them over all banks.
//    Every read address is one of 6 per-lane bases plus the slot base and a
//    constant in the instruction's offset field.
//  * The reads of a K slice are issued one half-stage ahead of its MFMAs,
//    interleaved with the MFMAs of the slice before (across the stage
//    barrier too), so the matrix cores do not wait for LDS after a barrier.
//  * The DMA is issued from inline asm and completion tracked with vmcnt, in
//    the same asm block as the barrier that publishes a stage (see dma.h).
// ---------------------------------------------------------------------------
constexpr int kDK = 32;                  // tokens per stage
constexpr int kDOpBytes = kDK * 512;     // one operand of one stage
constexpr int kDSlotBytes = 2 * kDOpBytes;

typedef int v4i32_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dma16_buf(uint32_t voff, v4i32_t rsrc, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds_base), "s"(soff) : "memory");
}

// WAVES = 4: one wave per SIMD, each a 128 x 128 block (2 x 2); WAVES = 8:
// two per SIMD, each 128 x 64 (2 x 4). SLOTS stages of kDK tokens are in
// the LDS ring (32 KiB each).
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait until at most `stages` stages of this wave's DMA (PER instructions
// each) are outstanding, then barrier (one asm block: no LDS read can be
// scheduled in between).
template <int PER, int MAXS>
__device__ __forceinline__ void wait_stages_barrier(int stages) {
  if (stages <= 0) wait_vm_barrier<0>();
  else if (stages == 1 || MAXS < 2) wait_vm_barrier<PER>();
  else if (stages == 2 || MAXS < 3) wait_vm_barrier<2 * PER>();
  else wait_vm_barrier<3 * PER>();
}

// Instruction scheduling groups for the compiler: one MFMA, then its share
// of NR LDS reads, NM times (the reads spread evenly over the MFMAs).
template <int NM, int NR, int I = 0>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int r = (I + 1) * NR / NM - I * NR / NM;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    sched_interleave<NM, NR, I + 1>();
  }
}

template <int WAVES, int SLOTS>
__global__ void __launch_bounds__(64 * WAVES)
k_hessian_dma(const uint16_t* __restrict__ X, int64_t T, int64_t n, int64_t ldx,
              float* __restrict__ part, int64_t chunk, int splits) {
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
  static_assert(SLOTS >= 3 && SLOTS <= 5, "3..5 slots");
  constexpr int PER = 32 / WAVES;         // DMA instructions per wave per stage
  constexpr int WN = WAVES / 2;           // waves across the columns
  constexpr int NB = 4 / (WN / 2);        // 32-column blocks per wave: 4 or 2
  __shared__ __align__(16) uint8_t dsm[SLOTS * kDSlotBytes];
  const int nt = (int)ceil_div(n, kHT);
  int tile, split, bi, bj;
  if (!hessian_item(blockIdx.x, nt * (nt + 1) / 2, splits, tile, split)) return;
  upper_tile(tile, nt, bi, bj);
  const int64_t kbeg = (int64_t)split * chunk;
  const int64_t kend = min(T, kbeg + chunk);
  const int64_t iA = (int64_t)bi * kHT, iB = (int64_t)bj * kHT;
  float* __restrict__ P = part + (int64_t)split * n * n;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dsm));

  // buffer over this chunk's tokens: [kbeg, kend) x ldx bf16
  v4i32_t rsrc;
  {
    const uint64_t base = (uint64_t)(uintptr_t)(X + kbeg * ldx);
    const int64_t bytes = kend > kbeg ? (kend - kbeg) * ldx * 2 : 0;
    rsrc.x = (int)(uint32_t)base;
    rsrc.y = (int)(uint32_t)(base >> 32);      // stride 0
    rsrc.z = (int)(uint32_t)bytes;             // the launcher keeps this below 2^31
    rsrc.w = 0x00020000;                       // raw buffer, 32-bit data format
    rsrc.x = __builtin_amdgcn_readfirstlane(rsrc.x);
    rsrc.y = __builtin_amdgcn_readfirstlane(rsrc.y);
    rsrc.z = __builtin_amdgcn_readfirstlane(rsrc.z);
  }
  // DMA plan: a stage is 2 operands x 16 row pairs = 32 wave-instructions;
  // wave w issues q = 0..PER-1 -> instruction PER w + q: operand idx / 16,
  // rows 2p, 2p+1 with p = idx % 16; lane l fills row 2p + l/32, slot chunk
  // l%32. A chunk past the last channel gets an offset beyond the buffer.
  uint32_t voff[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int idx = PER * wave + q;
    const int op = idx >> 4, p = idx & 15;
    const int t = 2 * p + (lane >> 5);
    const int c = (lane & 31) ^ dma_swz(t);
    const int64_t ch = (op ? iB : iA) + 8 * c;
    voff[q] = ch < n ? (uint32_t)((t * ldx + ch) * 2) : 0x80000000u;
  }
  const uint32_t stage_bytes = (uint32_t)(kDK * ldx * 2);
  // A diagonal tile needs one channel strip: the B operand is read from the
  // A region and its DMA is skipped (waves whose instructions are all B
  // then issue none; their stage waits are trivially met).
  const bool diag = bi == bj;
  auto issue = [&](int st, int slot) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)st * stage_bytes);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = PER * wave + q;
      const int op = idx >> 4, p = idx & 15;
      if (op == 1 && diag) continue;
      dma16_buf(voff[q], rsrc, soff,
                __builtin_amdgcn_readfirstlane(lds0 + slot * kDSlotBytes + op * kDOpBytes + p * 1024));
    }
  };

  // Transpose-read addresses (per lane, relative to a slot): group G =
  // lane/16, s = lane%16, token row t = 16 ks + 4 h + 8 (G/2) + s/4 and
  // chunk (c0 + 4 b + 2 (G%2) + (s/2)%2) ^ dma_swz(t), with c0 = 16 wm for
  // the A blocks b = 0..3 and c0 = 4 NB wn for the B blocks b < NB.
  const int G = lane >> 4, sl = lane & 15;
  const int trow_off = 8 * (G >> 1) + (sl >> 2);
  const int cbase = 2 * (G & 1) + ((sl >> 1) & 1);
  const int swz = dma_swz(trow_off);           // t % 4 == trow_off % 4
  const int half8 = (sl & 1) * 8;
  // per-lane read offsets of the A and B fragments at ks = 0, h = 0; a
  // stage adds its slot base once per fragment, and (ks, h) move by
  // constants that fit the instructions' 16-bit offset field
  uint32_t off[4 + NB];
#pragma unroll
  for (int b = 0; b < 4; ++b) off[b] = trow_off * 512 + (((16 * wm + 4 * b + cbase) ^ swz) * 16) + half8;
#pragma unroll
  for (int b = 0; b < NB; ++b)
    off[4 + b] = (diag ? 0 : kDOpBytes) + trow_off * 512 + (((4 * NB * wn + 4 * b + cbase) ^ swz) * 16) + half8;
  // on a diagonal tile, a wave whose block lies wholly below the diagonal
  // only takes part in the DMA and the barriers (that half is never read)
  const bool idle = diag && 4 * NB * wn * 8 + 32 * NB - 1 < 128 * wm;

  f32x16_t acc[4][NB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nstage = kend > kbeg ? (int)ceil_div(kend - kbeg, kDK) : 0;
#pragma unroll
  for (int ps = 0; ps < SLOTS - 1; ++ps)
    if (ps < nstage) issue(ps, ps);
  // the A / B operands of one 16-token K slice of the stage in `slot`
  auto read_slice = [&](int slot, int ks, bf16x8_t (&fa)[4], bf16x8_t (&fb)[NB]) {
    const uint32_t sbase = lds0 + (uint32_t)slot * kDSlotBytes + (uint32_t)(16 * ks) * 512;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const v4i16_t lo = lds_tr16(off[4 + b] + sbase), hi = lds_tr16(off[4 + b] + sbase + 2048);
      fb[b] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const v4i16_t lo = lds_tr16(off[b] + sbase), hi = lds_tr16(off[b] + sbase + 2048);
      fa[b] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mfma_slice = [&](const bf16x8_t (&fa)[4], const bf16x8_t (&fb)[NB]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
  };
  // Software pipeline across the stage barrier. The barrier that opens
  // stage st waits for the DMA of stages st and st + 1, so the first K slice
  // of stage st + 1 can be read during stage st: each half-stage issues the
  // MFMAs of one K slice interleaved with the reads of the next, and the
  // MFMAs after a barrier start on operands already in registers. The refill
  // issued after barrier st goes to the slot of stage st - 1, whose reads all
  // completed before its MFMAs (so no wave still reads a slot being filled);
  // the ring therefore runs SLOTS - 2 stages ahead. The last stage's read of
  // the next slot touches no slot being filled and is unused.
  bf16x8_t pa[4], pb[NB], qa[4], qb[NB];
  // 4 NB MFMAs and 2 (4 + NB) reads per half-stage
  auto interleave = [&]() { sched_interleave<4 * NB, 2 * (4 + NB)>(); };
  for (int st = 0; st < nstage; ++st) {
    const int pend = min(SLOTS - 3, nstage - 2 - st);
    wait_stages_barrier<PER, SLOTS - 3>(pend < 0 ? 0 : pend);
    if (st + SLOTS - 1 < nstage) issue(st + SLOTS - 1, (st + SLOTS - 1) % SLOTS);
    if (idle) continue;
    const int slot = st % SLOTS;
    if (st == 0) read_slice(slot, 0, pa, pb);
    __builtin_amdgcn_sched_barrier(0);
    read_slice(slot, 1, qa, qb);
    mfma_slice(pa, pb);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    read_slice(slot + 1 == SLOTS ? 0 : slot + 1, 0, pa, pb);
    mfma_slice(qa, qb);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  }

  if (idle) return;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = iA + 128 * wm + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t j = iB + 32 * NB * wn + 32 * nb + (lane & 31);
        if (i < n && j < n) P[i * n + j] = acc[mb][nb][r];
      }
}

constexpr int kDWaves = 8;
constexpr int kDSlotsUsed = 4;

hipError_t launch_hessian_partials_bf16(hipStream_t s, const uint16_t* X, int64_t T, int64_t n,
                                        int64_t ldx, float* part, int splits) {
  const int nt = (int)ceil_div(n, kHT);
  const int items = nt * (nt + 1) / 2 * splits;
  const int64_t chunk = ceil_div(ceil_div(T, splits), kHBK) * kHBK;
  const bool aligned = (n % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)X % 16 == 0);
  // 32-bit buffer offsets: a token chunk must span less than 2^31 bytes
  if (aligned && chunk * ldx * 2 < ((int64_t)1 << 31)) {
    const int64_t grid = 256 * (((int64_t)items + 255) / 256);   // whole rounds (hessian_item)
    hipLaunchKernelGGL((k_hessian_dma<kDWaves, kDSlotsUsed>), dim3((unsigned)grid), dim3(64 * kDWaves), 0,
                       s, X, T, n, ldx, part, chunk, splits);
  } else {
    hipLaunchKernelGGL(k_hessian_bf16<false>, dim3(items), dim3(256), 0, s, X, T, n, ldx, part, chunk);
  }
  return hipGetLastError();
}

hipError_t launch_hessian_partials_f32(hipStream_t s, const float* X, int64_t T, int64_t n,
                                       int64_t ldx, float* part, int splits) {
  const int64_t chunk = ceil_div(T, splits);
  for (int sp = 0; sp < splits; ++sp) {
    const int64_t kb = sp * chunk, ke = min(T, kb + chunk);
    GemmArgs g{};
    g.M = n; g.N = n; g.K = ke > kb ? ke - kb : 0;
    g.A = X + kb * ldx; g.lda = ldx; g.ta = 1;     // A(m,k) = X[k][m]
    g.B = X + kb * ldx; g.ldb = ldx; g.tb = 0;     // B(k,n) = X[k][n]
    g.C = part + (int64_t)sp * n * n; g.ldc = n;
    g.alpha = 1.f; g.beta = 0.f; g.kmode = 0; g.lower_only = 0;
    hipError_t e = launch_gemm_f32(s, g);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// H[i][j] (i <= j) = base + 2 * sum_s part[s][i][j]; H[j][i] = H[i][j].
// One 64x64 tile on or above the diagonal per workgroup; thread (ty, tx)
// sums rows ty + 16 q of columns 4 tx .. 4 tx + 3 with 16-byte loads when
// the row stride allows. The split count S is a template argument: a
// row's S loads are all issued before the sum (in split order, so the
// result is the same as a sequential sum), one memory round trip per row
// instead of one per split.
typedef float red_f32x4_t __attribute__((ext_vector_type(4)));

template <int S>
__global__ void __launch_bounds__(256)
k_hessian_reduce(const float* __restrict__ part, int64_t n, float* __restrict__ H, int zero_first) {
  constexpr int splits = S;
  __shared__ float tile[64][65];
  const int nt = (int)ceil_div(n, 64);
  int a, b;
  upper_tile(blockIdx.x, nt, a, b);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t nn = n * n;
  const int64_t j0 = (int64_t)b * 64 + 4 * tx;
  const bool vec = (n % 4 == 0) && (j0 + 3 < n);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = ty + 16 * q;
    const int64_t i = (int64_t)a * 64 + r;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (i < n) {
      if (vec) {
        red_f32x4_t x[S];
#pragma unroll
        for (int sp = 0; sp < S; ++sp) x[sp] = *reinterpret_cast<const red_f32x4_t*>(part + sp * nn + i * n + j0);
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int sp = 0; sp < S; ++sp) {
          sum.x += x[sp].x; sum.y += x[sp].y; sum.z += x[sp].z; sum.w += x[sp].w;
        }
        const float s4[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t jj = j0 + c;
          if (i <= jj) {
            v[c] = (zero_first ? 0.f : H[i * n + jj]) + 2.f * s4[c];
            H[i * n + jj] = v[c];
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t jj = j0 + c;
          if (jj < n && i <= jj) {
            float sum = 0.f;
            for (int sp = 0; sp < splits; ++sp) sum += part[sp * nn + i * n + jj];
            v[c] = (zero_first ? 0.f : H[i * n + jj]) + 2.f * sum;
            H[i * n + jj] = v[c];
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) tile[r][4 * tx + c] = v[c];
  }
  __syncthreads();
  // mirror: H[64b + r][64a + c] = tile[c][r] where (64a + c) < (64b + r)
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  for (int r = ry; r < 64; r += 4) {
    const int64_t i = (int64_t)b * 64 + r, jj = (int64_t)a * 64 + cx;
    if (i < n && jj < n && jj < i) H[i * n + jj] = tile[cx][r];
  }
}

template <int S>
static void launch_reduce_s(hipStream_t s, dim3 grid, const float* part, int64_t n, float* H, int zero_first) {
  hipLaunchKernelGGL(k_hessian_reduce<S>, grid, dim3(256), 0, s, part, n, H, zero_first);
}

template <int... Ss>
static bool launch_reduce_any(int splits, std::integer_sequence<int, Ss...>, hipStream_t s, dim3 grid,
                              const float* part, int64_t n, float* H, int zero_first) {
  return ((splits == Ss + 1 ? (launch_reduce_s<Ss + 1>(s, grid, part, n, H, zero_first), true) : false) || ...);
}

hipError_t launch_hessian_reduce(hipStream_t s, const float* part, int splits, int64_t n,
                                 float* H, int zero_first) {
  const int nt = (int)ceil_div(n, 64);
  const dim3 grid(nt * (nt + 1) / 2);
  // hessian_splits() returns 1..16
  if (!launch_reduce_any(splits, std::make_integer_sequence<int, 16>{}, s, grid, part, n, H, zero_first))
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gq
