// Grouped GEMM over the local experts for gfx950: the fused gate/up projection with SwiGLU, and
// the down projection.
//
// "Systems engineering playbook: optimizing Qwen 3.5-397B MoE on Ironwood (TPU7x)": the grouped
// GEMM building block (executive summary) over 64 local experts of intermediate size 1024
// (sections 1 and 3); decode batches stream every expert weight from HBM, prefill batches are
// bound by the matrix units (section 2).  "vLLM TPU Inference v0.31.0" (4-bit weight scope): int4
// weights stay packed in HBM and only the tiles in use are dequantised on chip.
//
// Design (MI355X):
//  - Work unit = tile (expert e, m-tile of BM rows of that expert, n-tile of BN output columns).
//    Tiles are numbered expert by expert, in groups of up to four m-tiles with the m-tile fastest,
//    so consecutive tiles reuse one weight slab and a few activation tiles.  Each workgroup derives the tile table from group_offsets in LDS, so
//    the number of local pairs never goes through the host.
//  - Persistent grid, a multiple of 8 workgroups.  Workgroup b runs on XCD b % 8; the tiles are
//    cut into 8 contiguous ranges and XCD x's workgroups walk range x, so tiles sharing a weight
//    slab or activation rows share one L2.
//  - Activation rows (gathered through row_index / row_div) and prepared dense weight rows
//    (W[e][n][k], K-contiguous: MOE_W_DENSE_NK) are copied into LDS the same way: 16 bytes per
//    lane, 8 lanes per 128-byte row chunk, giving [row][k] tiles whose rows are what the MFMA
//    operands read (8 consecutive k per lane).
//    int4 words [e][k/8][n] hold 8 consecutive k of one column: they are dequantised exactly to
//    fp16 into the same [n][k] LDS layout (each 16-byte chunk's eight k in the order the
//    dequantisation produces, the activations of those tiles reordered to match); fp8 bytes are
//    converted exactly to bf16 or fp16.
//  - 16x16x32 MFMA with fp32 accumulators; SwiGLU fused in the epilogue (each lane holds the gate
//    and the up value of the same output element).  Operands are bf16 (dense bf16 weights) or
//    fp16: int4 weights are dequantised exactly to fp16 (q * s has at most 11 significant bits;
//    a bf16 tile would round it), bf16 activations feeding them are converted to fp16 on their
//    way to LDS, and the down projection reads the fp16 SwiGLU output with fp16 weights.  fp16
//    weights carry a factor 2^8 that the epilogue removes.
//  - Decode-shaped tiles: global loads run ahead of the MFMAs through registers (two to four
//    chunks) into one or two LDS buffers.  Prefill-shaped dense tiles: chunks are copied global ->
//    LDS by the load unit (two or three buffers), or, for gate/up tiles whose weights no other
//    tile reads, the weights go through registers two chunks ahead.
#include "common.h"

namespace moe {
namespace {

struct GemmParams {
  const void* a;
  const int32_t* row_index;
  const int32_t* group_offsets;
  const void* w0;
  const void* w1;
  const void* s0;
  const void* s1;
  void* out;
  const float* bias;   // router logits: fp32 [N] added to each output row (or NULL)
  int K, N, n_groups, rows_cap, a_rows, row_div, group_size;
};

// ---------------------------------------------------------------------------------------------
// Tile table: s_tstart[e] = first tile of group e, s_tstart[n_groups] = total tiles;
// s_goff[e] = clamped row offset of group e.  Built by wave 0 in chunks of 64 groups.
// ---------------------------------------------------------------------------------------------
__device__ void build_tile_table(const GemmParams& p, int BM, int tiles_n, int* s_tstart, int* s_goff) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < p.n_groups; c0 += 64) {
    const int e = c0 + lane;
    int tiles = 0;
    if (e < p.n_groups) {
      // no group offsets: one group of rows_cap identity rows (the router projection)
      int lo = p.group_offsets ? p.group_offsets[e] : 0, hi = p.group_offsets ? p.group_offsets[e + 1] : p.rows_cap;
      lo = min(max(lo, 0), p.rows_cap);
      hi = min(max(hi, lo), p.rows_cap);
      s_goff[e] = lo;
      if (e == p.n_groups - 1) s_goff[p.n_groups] = hi;
      tiles = ((hi - lo + BM - 1) / BM) * tiles_n;
    }
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (e < p.n_groups) s_tstart[e] = carry + incl - tiles;
    carry += __shfl(incl, 63);
  }
  if (lane == 0) s_tstart[p.n_groups] = carry;
}

// Largest e with s_tstart[e] <= tile (groups with no tiles are skipped naturally).
__device__ __forceinline__ int find_group(const int* s_tstart, int n_groups, int tile) {
  int lo = 0, hi = n_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tstart[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct TileIter {
  int next, end, step;
};

struct TileCoord {
  int e, row0, rows, n0;
};

// Tile -> (expert, first output row, rows, first column).  Inside an expert, tiles go in groups
// of up to 4 m-tiles x all n-tiles, m-tile fastest: the workgroups of one XCD then share a few
// activation tiles and a few weight slabs in L2.
__device__ __forceinline__ TileCoord tile_coord(const int* s_tstart, const int* s_goff, int n_groups, int tile,
                                                int BM, int BN, int tiles_n) {
  constexpr int kGroupM = 4;
  const int e = find_group(s_tstart, n_groups, tile);
  const int g0 = s_goff[e], g1 = s_goff[e + 1];
  const int mtiles = (g1 - g0 + BM - 1) / BM;
  const int local = tile - s_tstart[e];
  const int grp = local / (kGroupM * tiles_n), in_grp = local % (kGroupM * tiles_n);
  const int gm = min(kGroupM, mtiles - grp * kGroupM);
  const int mt = grp * kGroupM + in_grp % gm, nt = in_grp / gm;
  const int row0 = g0 + mt * BM;
  return {e, row0, min(BM, g1 - row0), nt * BN};
}

// XCD-aware static schedule over [0, total).
__device__ __forceinline__ TileIter tile_range(int total) {
  const int G = gridDim.x;               // a multiple of 8
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3, gx = G >> 3;
  const int per = (total + 7) >> 3;
  const int beg = xcd * per;
  return {beg + j, min(total, beg + per), gx};
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return __fdividef(g, 1.0f + __expf(-g)) * u;
}

// One 16x16x32 MFMA on 16-byte operand registers: bf16 or fp16 inputs, fp32 accumulation.
template <bool F16>
__device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
}

// Output element stores: fp32, bf16 (u16 bits) or fp16, rounded to nearest even.
template <typename OutT>
__device__ __forceinline__ void store_out(OutT* dst, float v) {
  if constexpr (sizeof(OutT) == 4) *dst = v;
  else if constexpr (__is_same(OutT, _Float16)) *dst = (_Float16)v;
  else *dst = f32_to_bf16(v);
}

// ---------------------------------------------------------------------------------------------
// MFMA kernel with register-staged loads
// ---------------------------------------------------------------------------------------------
constexpr size_t kLdsPerCu = 160 * 1024;             // LDS of one gfx950 compute unit

// Raw buffer resource (gfx9 family dword 3): weight loads use one scalar descriptor per tile
// plus 32-bit per-lane byte offsets.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// F16_: fp16 MFMA operands (weights scaled by 2^8); ACVT_: the activation matrix is bf16 and is
// converted to fp16 on its way to LDS.  int4 weights always run on fp16 operands.
// SUM_ (with GU_): the epilogue writes acc0 + acc1 (+ bias) in fp32 instead of SwiGLU: the router
// projection over an fp32 weight split into two bf16 planes.
// W8_: fp8 (e4m3) weights [e][N][K], converted exactly to the operand type (bf16 or fp16) on their
// way to LDS, with one scale per output column applied in the epilogue.
// KN_: dense bf16 weights in the stated [e][K][N] layout (each K row's N weights contiguous): K
// rows go to LDS as they are and the MFMA B operands are read transposed (ds_read_b64_tr_b16).
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, bool GU_, bool Q4_, int WGS_ = 1, int REGSETS_ = 2,
          bool F16_ = Q4_, bool ACVT_ = false, bool SUM_ = false, bool W8_ = false, bool KN_ = false>
struct Cfg {
  static constexpr bool F16 = F16_, ACVT = ACVT_, SUM = SUM_, W8 = W8_, KN = KN_;
  // fp16 operands carry weights scaled by 2^8 (int4, prepared dense fp16), fp8 ones do not
  static constexpr float OUT_MUL = (F16_ && !W8_) ? 1.0f / kF16WeightScale : 1.0f;
  // Chunks held in registers between their loads and their LDS stores (two LDS buffers only).
  static constexpr int REGSETS = REGSETS_;
  // fp8 decode tiles (four chunks in registers) load two chunks of a column at once: 128
  // contiguous bytes, a whole cache line, instead of two halves a chunk apart (gate/up 127 -> 91
  // us, down 69 -> 56 us at the decode shape, with compact addressing that does not spill).
  static constexpr bool W8PAIR = W8_ && REGSETS_ == 4;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
  static constexpr int WGS = WGS_;                  // intended workgroups per CU
  static constexpr int WAVES_PER_SIMD = (WM_ * WN_ * WGS_ + 3) / 4;   // register budget target
  static constexpr bool GU = GU_, Q4 = Q4_;
  static constexpr int NWAVES = WM * WN, NT = 64 * NWAVES;    // threads per workgroup
  static constexpr int KC = 64;                     // K chunk per LDS stage
  static constexpr int NW = GU ? 2 : 1;             // weight matrices
  static constexpr int LDK = KC;                    // LDS row: 64 bf16 = 128 bytes, 16-byte chunks swizzled
  static constexpr int A_ELEMS = BM * LDK;
  static constexpr int B_ELEMS = NW * BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;   // u16 elements per LDS buffer
  static constexpr int A_CHUNKS = BM * (KC / 8);    // 16-byte pieces of the A tile
  static constexpr int A_LOADS = A_CHUNKS >= NT ? A_CHUNKS / NT : 1;   // per thread (small tiles: duplicated)
  // B units per thread: a dense R x 8 block or one 16-byte row of 4 int4 words, 32 weights each
  static constexpr int B_UNITS = NW * KC * BN / 32 / NT;
  static constexpr int R = 4;                       // dense: 16-byte pieces per unit
  static constexpr int B_PIECES = B_UNITS * R;      // dense: 16-byte pieces per thread
  static constexpr int SLICE_ROWS = NT / 8;         // 128-byte rows filled by one 16-byte piece per thread
  static constexpr int NRSRC = B_UNITS > NW ? B_UNITS : NW;
  static constexpr int MT = BM / WM / 16;           // 16-row MFMA tiles per wave
  static constexpr int NTL = BN / WN / 16;          // 16-column MFMA tiles per wave and matrix
  static_assert(NWAVES == 4 || NWAVES == 8, "four or eight waves");
  static_assert(STAGES == 1 || STAGES == 2, "LDS buffers");
  static_assert(REGSETS == 2 || (REGSETS == 1 && STAGES == 2) || (REGSETS == 4 && STAGES == 1), "register sets");
  static_assert(A_CHUNKS % NT == 0 || NT % A_CHUNKS == 0, "A tile split");
  static_assert(B_UNITS >= 1 && (NW * KC * BN) % (32 * NT) == 0, "B tile split");
  static_assert(MT >= 1 && NTL >= 1, "wave tile");
  static_assert(Q4 || BN % SLICE_ROWS == 0, "a dense piece slice stays inside one weight matrix");
  static_assert(!Q4 || F16, "int4 weights are dequantised to fp16");
  static_assert(!W8_ || !ACVT, "fp8 weights convert to the activations' 16-bit type");
  static_assert(!ACVT || F16, "activations are converted to the fp16 operand type");
  static_assert(!SUM || (GU && !Q4 && !F16 && !W8_), "router sums: two dense bf16 weight planes");
  static_assert(!(Q4 && W8_), "one weight format");
  static_assert(!KN_ || (!Q4 && !W8_ && !F16 && (BN == 64 || BN == 128)), "[K][N] tiles: bf16, 64 or 128 columns");
  static size_t lds_bytes(int n_groups) { return STAGES * STAGE * 2 + 2 * sizeof(int) * (n_groups + 1) + 16; }
};

// LDS tiles hold one 128-byte row (64 consecutive k) per activation row or weight column, in
// 16-byte chunks; chunk q of row n sits at position q ^ swz(n) with swz(n) = (n/2) mod 8.  The MFMA
// operand reads (16 consecutive rows, one chunk per 16-lane group) are free of bank conflicts
// because swz runs over 0..7 on the even and on the odd rows of every 16-row block, and since swz
// depends on n mod 16 only, all operand reads of a lane are one base register plus immediate
// offsets.  Dequantised int4 columns are written so that each 16-lane pass fills 8 chunks of an
// even row and 8 of an odd row (see the int4 unit mapping), also without conflicts.
__device__ __forceinline__ int lds_off_rows(int n, int q) { return n * 64 + ((q ^ ((n >> 1) & 7)) << 3); }

// [K][N] weight tiles hold one row of BN columns per k (BN / 8 chunks of 16 bytes); chunk c of row
// k sits at position c ^ swz_kn(k).  A transposed operand read by 32 lanes touches 8 rows (k and
// k + 8 blocks of 4) and 2 chunks in each; swz_kn sends them to 16 different 16-byte bank slots
// (rows of 256 bytes fill all 64 banks, rows of 128 bytes half of them, alternating).  Within a
// lane's operand reads swz_kn depends only on the lane, so each read is one base plus offsets.
template <int BN>
__device__ __forceinline__ int swz_kn(int k) {
  if constexpr (BN == 128) return 2 * ((k & 3) + 4 * ((k >> 3) & 1));
  else return 2 * (((k >> 1) & 1) + 2 * ((k >> 3) & 1));
}

// Registers holding one K chunk in flight: the activation rows and the weight units of this
// thread.
template <class C>
struct AChunk {
  u32x4 a[C::A_LOADS];
};
template <class C>
struct WChunk {
  u32x4 b[C::B_UNITS][C::Q4 ? 1 : (C::W8 ? 2 : C::R)];   // int4: 4 words; fp8: two 16-byte pieces; dense: R pieces
  u32x2 s[C::B_UNITS];
};
template <class C>
struct Chunk {
  AChunk<C> a;
  WChunk<C> w;
};

// Everything a thread needs to move one tile's chunks: gathered A row pointers, the weight and
// scale descriptors of the tile's expert and its own byte offsets, and LDS destinations.
template <class C>
struct TileCtx {
  __amdgpu_buffer_rsrc_t ar;                        // activation matrix
  uint32_t a_off[C::A_LOADS];                       // byte offset of the lane's piece of chunk 0
  int a_lds;                                        // LDS destination of the lane's first piece
  __amdgpu_buffer_rsrc_t wr[C::NRSRC];           // dense: one per matrix; int4: one per unit
  __amdgpu_buffer_rsrc_t sr[C::B_UNITS];
  uint32_t b_voff;                                  // dense: lane offset (row lane/8, chunk lane%8)
  uint32_t b_soff;                                  // dense: wave-uniform offset of the wave's rows
  int b_lds;                                        // dense: LDS destination of the lane's first piece
  uint32_t b_off[C::B_UNITS];                       // int4: word offset of the unit
  uint32_t s_off[C::B_UNITS];                       // int4: scale offset of the unit
  uint32_t kn_voff[C::KN ? C::B_PIECES : 1];        // [K][N]: lane offset of each 16-byte piece (row k, chunk c)
  int kn_dst[C::KN ? C::B_PIECES : 1];              // [K][N]: LDS destination of each piece
  int kn_m[C::KN ? C::B_PIECES : 1];                // [K][N]: matrix of each piece (wave-uniform)
  uint32_t kn_soff;                                 // [K][N]: byte offset of the tile's first column
  int b_dst[C::B_UNITS][C::Q4 ? 4 : (C::W8 ? 8 : 1)];   // int4: LDS destination of each dequantised column;
                                                    // fp8: of each 16-byte LDS chunk (two per piece)
  uint32_t w8_off[C::W8 ? 4 * C::B_UNITS : 1];      // fp8: byte offset of each piece in chunk 0
  int w8_m[C::W8 ? 4 * C::B_UNITS : 1];             // fp8: matrix of each piece (wave-uniform)
  bool w8_hi;                                       // fp8 pairs: the lane's pieces are the pair's second chunk
  bool b_swap[C::B_UNITS];                          // int4: columns written in swapped pairs
  const u16* es[C::NW];                             // fp8: scales of the tile's first column, per matrix
  int nK, row_bytes, s_row_bytes, group_size;
};

// Loads are unconditional (indices clamped to the last chunk): a branch around a load would make
// the compiler wait for every outstanding load, including the chunks prefetched ahead.
template <class C>
__device__ __forceinline__ void load_a(const TileCtx<C>& t, int kc, AChunk<C>& ch) {
  kc = min(kc, t.nK - 1);
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i)
    ch.a[i] = __builtin_amdgcn_raw_buffer_load_b128(t.ar, t.a_off[i], (uint32_t)kc * (C::KC * 2), 0);
}

template <class C>
__device__ __forceinline__ void load_w(const TileCtx<C>& t, int kc, WChunk<C>& ch) {
  kc = min(kc, t.nK - 1);
  if constexpr (C::KN) {
    // [K][N]: piece x is 8 consecutive columns of one K row of the chunk
    const uint32_t so = t.kn_soff + (uint32_t)kc * C::KC * t.row_bytes;
#pragma unroll
    for (int x = 0; x < C::B_PIECES; ++x) {
      __amdgpu_buffer_rsrc_t w = t.wr[0];
      if constexpr (C::NW == 2) w = t.kn_m[x] ? t.wr[1] : t.wr[0];
      ch.b[x / C::R][x % C::R] = __builtin_amdgcn_raw_buffer_load_b128(w, t.kn_voff[x], so, 2);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::B_UNITS; ++i) {
    if constexpr (C::W8) {
      // two pieces of 16 consecutive k of one column each: K bytes per column, the chunk at byte
      // kc * 64
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        __amdgpu_buffer_rsrc_t w = t.wr[0];
        if constexpr (C::NW == 2) w = t.w8_m[2 * i + h] ? t.wr[1] : t.wr[0];
        ch.b[i][h] = __builtin_amdgcn_raw_buffer_load_b128(w, t.w8_off[2 * i + h] + (uint32_t)kc * C::KC, 0, 2);
      }
    } else if constexpr (!C::Q4) {
      // piece x = i*R + r covers weight rows SLICE_ROWS*x .. SLICE_ROWS*(x+1)-1 of the NW*BN tile rows
#pragma unroll
      for (int r = 0; r < C::R; ++r) {
        const int x = i * C::R + r;
        const int rows_x = C::SLICE_ROWS * x;
        const uint32_t so = t.b_soff + (uint32_t)(rows_x % C::BN) * t.row_bytes + (uint32_t)kc * (C::KC * 2);
        ch.b[i][r] = __builtin_amdgcn_raw_buffer_load_b128(t.wr[rows_x / C::BN], t.b_voff, so, 2 /* nontemporal */);
      }
    } else {
      ch.b[i][0] = __builtin_amdgcn_raw_buffer_load_b128(
          t.wr[i], t.b_off[i] + (uint32_t)(kc * (C::KC / 8)) * t.row_bytes, 0, 2);
      // the scale group of this unit's word row, (kc * 64 + k) / group_size: the chunk's first
      // group (kc * 64) / group_size, exact for group sizes that divide 64 or are multiples of it,
      // plus the word row's group inside the chunk (nonzero below 64), which s_off holds
      const int grp = (kc * C::KC) / t.group_size;
      ch.s[i] = __builtin_amdgcn_raw_buffer_load_b64(t.sr[i], t.s_off[i] + (uint32_t)grp * t.s_row_bytes, 0, 0);
    }
  }
}

// bf16 -> fp16 of eight packed values (exact for magnitudes in fp16's normal range).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4& v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_f16x2(__uint_as_float(v[i] << 16), __uint_as_float(v[i] & 0xffff0000u));
  return r;
}

// int4 tiles hold the eight k of each 16-byte LDS chunk, activations and weights alike, in the
// order k0 k4 k1 k5 k2 k6 k3 k7: the order in which the int4 dequantisation below produces them
// with the fewest instructions.  An MFMA multiplies the operand elements of equal position, so
// equal permutations of both operands leave every product, and the sum over the chunk, the same.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_il(const u32x4& v) {
  return u32x4{pack_f16x2(__uint_as_float(v[0] << 16), __uint_as_float(v[2] << 16)),
               pack_f16x2(__uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[2] & 0xffff0000u)),
               pack_f16x2(__uint_as_float(v[1] << 16), __uint_as_float(v[3] << 16)),
               pack_f16x2(__uint_as_float(v[1] & 0xffff0000u), __uint_as_float(v[3] & 0xffff0000u))};
}
__device__ __forceinline__ u32x4 f16x8_il(const u32x4& v) {
  // v_perm_b32 byte selectors: 0-3 pick bytes of the second operand, 4-7 of the first
  return u32x4{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u), __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
               __builtin_amdgcn_perm(v[3], v[1], 0x05040100u), __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
}

template <class C>
__device__ __forceinline__ void store_a(const TileCtx<C>& t, const AChunk<C>& ch, u16* buf) {
  u16* sA = buf;
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    u32x4 v = ch.a[i];
    if constexpr (C::Q4) v = C::ACVT ? bf16x8_to_f16x8_il(v) : f16x8_il(v);
    else if constexpr (C::ACVT) v = bf16x8_to_f16x8(v);
    *reinterpret_cast<u32x4*>(sA + t.a_lds + C::SLICE_ROWS * i * 64) = v;
  }
}

// Eight int4 weights (the nibbles of one word, k ascending) times their scale, exactly, as eight
// fp16 values in the int4 tiles' order k0 k4 | k1 k5 | k2 k6 | k3 k7.  Nibble u (two's complement
// q) -> u ^ 8 = q + 8.  Masking the word with 0x000f000f (nibbles 0 and 4) and setting the
// exponent bits of 1024 in both halves gives the fp16 pair 1032 + q; with 0x00f000f0 (nibbles 1
// and 5) the nibble sits four bits higher, 1024 + 16 (q + 8), and times 1/16 minus 72 leaves q.
// The word shifted down by 8 bits gives nibbles 2, 6 and 3, 7 the same way.  Each step is exact
// in fp16 (all values are integers below 2048), and q * (s * 2^8) has at most 3 + 8 significant
// bits, so the packed fp16 product is exact.
__device__ __forceinline__ u32x4 dequant_int4_f16(uint32_t word, f16x2 scale2) {
  const uint32_t x = word ^ 0x88888888u, y = x >> 8;
  const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2 inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2 bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const f16x2 q0 = __builtin_bit_cast(f16x2, (x & 0x000f000fu) | 0x64006400u) + bias;
  const f16x2 q1 = __builtin_bit_cast(f16x2, (x & 0x00f000f0u) | 0x64006400u) * inv16 + bias16;
  const f16x2 q2 = __builtin_bit_cast(f16x2, (y & 0x000f000fu) | 0x64006400u) + bias;
  const f16x2 q3 = __builtin_bit_cast(f16x2, (y & 0x00f000f0u) | 0x64006400u) * inv16 + bias16;
  return u32x4{__builtin_bit_cast(uint32_t, q0 * scale2), __builtin_bit_cast(uint32_t, q1 * scale2),
               __builtin_bit_cast(uint32_t, q2 * scale2), __builtin_bit_cast(uint32_t, q3 * scale2)};
}

// bf16 scale bits -> fp16 pair of the scale times 2^8 (exact for 2^-22 <= s < 32)
__device__ __forceinline__ f16x2 scale_f16x2(uint32_t sbits) {
  const _Float16 h = (_Float16)(__uint_as_float(sbits << 16) * kF16WeightScale);
  return f16x2{h, h};
}

// Four fp8 values (one dword, k ascending) -> two dwords of 16-bit operands, exactly (e4m3's 4
// significant bits and exponent range fit bf16 and fp16).
template <bool F16>
__device__ __forceinline__ u32x2 fp8x4_to_16(uint32_t d) {
  if constexpr (F16)
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true))};
  else
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, true))};
}

template <class C>
__device__ __forceinline__ void store_w(const TileCtx<C>& t, const WChunk<C>& ch, u16* buf) {
  u16* sB = buf + C::A_ELEMS;
  if constexpr (C::KN) {
#pragma unroll
    for (int x = 0; x < C::B_PIECES; ++x) *reinterpret_cast<u32x4*>(sB + t.kn_dst[x]) = ch.b[x / C::R][x % C::R];
    return;
  }
#pragma unroll
  for (int i = 0; i < C::B_UNITS; ++i) {
    if constexpr (C::W8) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {                  // eight k per 16-byte LDS chunk
        const u32x2 lo = fp8x4_to_16<C::F16>(ch.b[i][c >> 1][2 * (c & 1)]);
        const u32x2 hi = fp8x4_to_16<C::F16>(ch.b[i][c >> 1][2 * (c & 1) + 1]);
        *reinterpret_cast<u32x4*>(sB + t.b_dst[i][c]) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    } else if constexpr (!C::Q4) {
#pragma unroll
      for (int r = 0; r < C::R; ++r)
        *reinterpret_cast<u32x4*>(sB + t.b_lds + C::SLICE_ROWS * (i * C::R + r) * 64) = ch.b[i][r];
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // column c of the unit, or c ^ 1 for units written in swapped pairs
        const uint32_t word = t.b_swap[i] ? ch.b[i][0][c ^ 1] : ch.b[i][0][c];
        const uint32_t sdw = ch.s[i][c >> 1];
        const uint32_t sbits = ((c & 1) != (int)t.b_swap[i]) ? (sdw >> 16) : (sdw & 0xffffu);
        *reinterpret_cast<u32x4*>(sB + t.b_dst[i][c]) = dequant_int4_f16(word, scale_f16x2(sbits));
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void load_chunk(const TileCtx<C>& t, int kc, Chunk<C>& ch) {
  load_a(t, kc, ch.a);
  load_w(t, kc, ch.w);
}

// fp8 chunk pairs: chunks kc (even) and kc + 1 of the activation rows, and the pair's weight
// pieces (128 bytes of each column), pieces 0, 1 of each unit into e, 2, 3 into o.
template <class C>
__device__ __forceinline__ void load_pair(const TileCtx<C>& t, int kc, Chunk<C>& e, Chunk<C>& o) {
  kc = min(kc, t.nK - 2);
  load_a(t, kc, e.a);
  load_a(t, kc + 1, o.a);
#pragma unroll
  for (int i = 0; i < C::B_UNITS; ++i)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      constexpr int PC = C::NT / 8;                 // columns per piece load of the workgroup
      const int q = 4 * i + x;
      const int mq = (PC * q) / C::BN, cq = (PC * q) % C::BN;   // matrix and first column of piece q
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(t.wr[mq], t.w8_off[0] + (uint32_t)(cq * t.row_bytes) +
                                                            (uint32_t)kc * C::KC, 0, 2);
      if (x < 2) e.w.b[i][x] = v;
      else o.w.b[i][x - 2] = v;
    }
}

// Chunk kc of a pair: its activation rows, and the weight pieces of the lanes that hold this
// chunk (the first or second 64 bytes of their column's 128); the other lanes store no weights.
template <class C>
__device__ __forceinline__ void store_pair_chunk(const TileCtx<C>& t, const Chunk<C>& ch, const Chunk<C>& e,
                                                 const Chunk<C>& o, bool second, u16* buf) {
  store_a(t, ch.a, buf);
  if (t.w8_hi != second) return;
  u16* sB = buf + C::A_ELEMS;
#pragma unroll
  for (int i = 0; i < C::B_UNITS; ++i)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      constexpr int PC = C::NT / 8;
      const int q = 4 * i + x;
      const int row = (PC * q) / C::BN * C::BN + (PC * q) % C::BN;   // first tile row of piece q
      const u32x4 v = x < 2 ? e.w.b[i][x] : o.w.b[i][x - 2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {                  // eight k per 16-byte LDS chunk
        const u32x2 lo = fp8x4_to_16<C::F16>(v[2 * c]);
        const u32x2 hi = fp8x4_to_16<C::F16>(v[2 * c + 1]);
        *reinterpret_cast<u32x4*>(sB + t.b_dst[0][c] + row * 64) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
}

template <class C>
__device__ __forceinline__ void store_chunk(const TileCtx<C>& t, const Chunk<C>& ch, u16* buf) {
  store_a(t, ch.a, buf);
  store_w(t, ch.w, buf);
}

// B operand of one 16x16x32 MFMA from a [K][N] tile: lanes 16 g .. 16 g + 15 need k = ks + 8 g ..
// + 7 of columns ncol .. ncol + 15.  ds_read_b64_tr_b16 gives lane i of a 16-lane group the
// (i % 4)-th 16-bit value of the 8 bytes addressed by lane 4 j + i / 4 as its value j, so lane L
// addresses columns ncol + 4 (L % 4) .. + 3 of row k0 + L / 4; two reads cover k0 = 8 g and 8 g + 4.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
template <class C>
__device__ __forceinline__ u32x4 read_kn_operand(const u16* sB, int m, int ks, int ncol) {
  const int lane = threadIdx.x & 63, L = lane & 15, g = lane >> 4;
  const int k = ks + 8 * g + (L >> 2);
  const int c = (ncol >> 3) + ((L & 3) >> 1);
  const int off = m * C::BN * C::KC + k * C::BN + ((c ^ swz_kn<C::BN>(k)) << 3) + 4 * (L & 1);
  const bf16x4_t* p0 = reinterpret_cast<const bf16x4_t*>(sB + off);
  const bf16x4_t* p1 = reinterpret_cast<const bf16x4_t*>(sB + off + 4 * C::BN);   // k + 4 (same swizzle)
  typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
  const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
  const u32x2 a = __builtin_bit_cast(u32x2, v0), b = __builtin_bit_cast(u32x2, v1);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// MFMAs of one LDS chunk for the NM live 16-row tiles of this wave (tile i covers rows
// arow0 - lane%16 + 16 * WM * i: the 16-row tiles of a workgroup tile are dealt to its WM wave
// rows in turn, which balances partially filled tiles).
template <class C, int NM, int NA = (NM > 0 ? NM : 1)>
__device__ __forceinline__ void compute_chunk(const u16* buf, f32x4 (&acc)[C::NW][NA][C::NTL],
                                              int arow, int bcol, int kofs) {
  if constexpr (NM > 0) {
    const u16* sA = buf;
    const u16* sB = buf + C::A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < C::KC; ks += 32) {
      u32x4 av[NM];
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const int off = lds_off_rows(arow, (ks + kofs) >> 3) + i * 16 * C::WM * 64;
        av[i] = *reinterpret_cast<const u32x4*>(sA + off);
      }
#pragma unroll
      for (int m = 0; m < C::NW; ++m) {
#pragma unroll
        for (int j = 0; j < C::NTL; ++j) {
          u32x4 bv;
          if constexpr (C::KN) {
            bv = read_kn_operand<C>(sB, m, ks, bcol - (bcol & 15) + j * 16);
          } else {
            const int off = lds_off_rows(bcol, (ks + kofs) >> 3) + (m * C::BN + j * 16) * 64;
            bv = *reinterpret_cast<const u32x4*>(sB + off);
          }
#pragma unroll
          for (int i = 0; i < NM; ++i) acc[m][i][j] = mma<C::F16>(av[i], bv, acc[m][i][j]);
        }
        // int4 prefill tiles: the operand reads of the next matrix and k-step stay behind these
        // MFMAs (hoisted, they would hold more operand registers next to the dequantised chunk's)
        if constexpr (C::Q4 && C::NWAVES == 8) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// K loop and epilogue of one tile for a wave with NM live 16-row tiles.  Every wave runs the same
// loads, LDS stores and barriers whatever its NM.
template <class C, typename OutT, int NM>
__device__ __forceinline__ void tile_body(const TileCtx<C>& t, u16* buf0, u16* buf1, OutT* O, int N, int lane,
                                          int wrow0, int wcol0, int row0, int rows, int n0, const float* bias) {
  f32x4 acc[C::NW][NM > 0 ? NM : 1][C::NTL];
#pragma unroll
  for (int m = 0; m < C::NW; ++m)
#pragma unroll
    for (int i = 0; i < (NM > 0 ? NM : 1); ++i)
#pragma unroll
      for (int j = 0; j < C::NTL; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int arow = wrow0 + (lane & 15);
  const int bcol = wcol0 + (lane & 15);
  const int kofs = (lane >> 4) * 8;
  const int nK = t.nK;

  // Loads run two chunks ahead of the MFMAs (two register sets).  With two LDS buffers one
  // barrier per chunk suffices; with one buffer it is refilled between two barriers.
  int kc = 0;
  if constexpr (C::STAGES == 2 && C::REGSETS == 1) {
    // One register set: a chunk's loads are issued right after the previous chunk is stored and
    // have one chunk of MFMAs (and the other waves of the SIMD) to arrive.
    Chunk<C> c0;
    load_chunk(t, 0, c0);
    store_chunk(t, c0, buf0);
    load_chunk(t, 1, c0);
    __syncthreads();
    for (; kc + 1 < nK; kc += 2) {
      compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
      store_chunk(t, c0, buf1);
      load_chunk(t, kc + 2, c0);
      __syncthreads();
      compute_chunk<C, NM>(buf1, acc, arow, bcol, kofs);
      store_chunk(t, c0, buf0);
      load_chunk(t, kc + 3, c0);
      __syncthreads();
    }
    if (kc < nK) compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
  } else if constexpr (C::STAGES == 2) {
    Chunk<C> c0, c1;
    load_chunk(t, 0, c0);
    load_chunk(t, 1, c1);
    store_chunk(t, c0, buf0);
    load_chunk(t, 2, c0);
    __syncthreads();
    for (; kc + 1 < nK; kc += 2) {                 // straight-line body: chunks kc and kc + 1
      compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
      store_chunk(t, c1, buf1);
      load_chunk(t, kc + 3, c1);
      __syncthreads();
      compute_chunk<C, NM>(buf1, acc, arow, bcol, kofs);
      store_chunk(t, c0, buf0);
      load_chunk(t, kc + 4, c0);
      __syncthreads();
    }
    if (kc < nK) compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
  } else if constexpr (C::REGSETS == 4) {
    // One LDS buffer, RS = 4 chunks in registers (the caller keeps K a multiple of RS chunks):
    // the quantised weights carry half or a quarter of the bytes of a 16-bit chunk, so a
    // decode-shaped tile keeps more chunks in flight to hold more bytes in flight.  The prologue
    // issues the chunks in the loop's order: the wait at the loop head covers the oldest chunk on
    // both entry edges only when they leave the loads in the same order (else the head waits for
    // every load in flight, once per RS chunks).
    constexpr int RS = C::REGSETS;
    Chunk<C> c[RS];
    if constexpr (C::W8PAIR) {
      // fp8: chunks loaded in pairs (one 128-byte line per column), a pair issued once both of
      // its register sets are stored
#pragma unroll
      for (int r = 0; r < RS; r += 2) {
        load_pair(t, r, c[r], c[r + 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (; kc < nK; kc += RS) {
#pragma unroll
        for (int r = 0; r < RS; ++r) {
          store_pair_chunk(t, c[r], c[r & ~1], c[r | 1], (r & 1) != 0, buf0);
          __syncthreads();
          compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
          if (r & 1) load_pair(t, kc + RS + r - 1, c[r - 1], c[r]);   // clamped past the end
          __syncthreads();
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        load_chunk(t, r, c[r]);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (; kc < nK; kc += RS) {
#pragma unroll
        for (int r = 0; r < RS; ++r) {
          store_chunk(t, c[r], buf0);
          __syncthreads();
          compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
          load_chunk(t, kc + RS + r, c[r]);                // clamped past the end
          __syncthreads();
        }
      }
    }
  } else {
    Chunk<C> c0, c1;
    load_chunk(t, 0, c0);
    load_chunk(t, 1, c1);
    // The next loads are issued after the MFMAs: when the vector L1 has no room for more misses
    // a load blocks the wave at issue, and it must not hold back the MFMAs.
    for (; kc + 1 < nK; kc += 2) {
      store_chunk(t, c0, buf0);
      __syncthreads();
      compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
      load_chunk(t, kc + 2, c0);
      __syncthreads();
      store_chunk(t, c1, buf0);
      __syncthreads();
      compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
      load_chunk(t, kc + 3, c1);
      __syncthreads();
    }
    if (kc < nK) {
      store_chunk(t, c0, buf0);
      __syncthreads();
      compute_chunk<C, NM>(buf0, acc, arow, bcol, kofs);
    }
  }
  __syncthreads();                                 // LDS is refilled by the next tile

  // epilogue: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16 tile
#pragma unroll
  for (int i = 0; i < NM; ++i)
#pragma unroll
    for (int j = 0; j < C::NTL; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wrow0 + i * 16 * C::WM + (lane >> 4) * 4 + r;
        const int col = wcol0 + j * 16 + (lane & 15);
        if (row < rows) {
          float m0 = C::OUT_MUL, m1 = C::OUT_MUL;
          if constexpr (C::W8) {                     // fp8: the output column's scales
            m0 = bf16_to_f32(t.es[0][col]);
            if constexpr (C::NW == 2) m1 = bf16_to_f32(t.es[C::NW - 1][col]);
          }
          float v;
          if constexpr (C::SUM) {
            v = acc[0][i][j][r] + acc[1][i][j][r];
            if (bias) v = v + bias[n0 + col];
          } else if constexpr (C::GU) {
            v = silu_mul(acc[0][i][j][r] * m0, acc[1][i][j][r] * m1);
          } else {
            v = acc[0][i][j][r] * m0;
          }
          store_out(O + (size_t)(row0 + row) * N + n0 + col, v);
        }
      }
}

template <class C, typename OutT, int NM>
__device__ __forceinline__ void tile_dispatch(int nm, const TileCtx<C>& t, u16* buf0, u16* buf1, OutT* O, int N,
                                              int lane, int wrow0, int wcol0, int row0, int rows, int n0,
                                              const float* bias) {
  if constexpr (NM <= C::MT) {
    if (nm == NM) tile_body<C, OutT, NM>(t, buf0, buf1, O, N, lane, wrow0, wcol0, row0, rows, n0, bias);
    else tile_dispatch<C, OutT, NM + 1>(nm, t, buf0, buf1, O, N, lane, wrow0, wcol0, row0, rows, n0, bias);
  }
}

template <class C, typename OutT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_SIMD)))
void k_gemm_bf16(GemmParams p) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, KC = C::KC, NT = C::NT;
  extern __shared__ __attribute__((aligned(16))) u16 smem[];
  u16* buf0 = smem;
  u16* buf1 = smem + (C::STAGES - 1) * C::STAGE;
  int* s_tstart = reinterpret_cast<int*>(smem + C::STAGES * C::STAGE);
  int* s_goff = s_tstart + (p.n_groups + 1);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = p.N / BN;
  const int wrow0 = wm * 16, wcol0 = wn * (BN / WN);

  build_tile_table(p, BM, tiles_n, s_tstart, s_goff);
  __syncthreads();
  const int total = s_tstart[p.n_groups];
  const TileIter it = tile_range(total);

  // the host checks a_rows * K * 2 < 2^32
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.a, (uint32_t)((size_t)p.a_rows * p.K * 2));
  OutT* O = static_cast<OutT*>(p.out);
  const uint32_t w_bytes = C::Q4 ? (uint32_t)((size_t)p.K / 8 * p.N * 4)
                                 : (uint32_t)((size_t)p.K * p.N * (C::W8 ? 1 : 2));
  const uint32_t s_bytes = C::Q4 ? (uint32_t)((size_t)(p.K / p.group_size) * p.N * 2) : 0u;

  for (int tile = it.next; tile < it.end; tile += it.step) {
    const TileCoord tc = tile_coord(s_tstart, s_goff, p.n_groups, tile, BM, BN, tiles_n);
    const int e = tc.e, row0 = tc.row0, rows = tc.rows, n0 = tc.n0;
    const int nm = min(C::MT, max(0, ((rows + 15) / 16 - wm + WM - 1) / WM));   // live 16-row tiles

    TileCtx<C> t;
    t.ar = a_rsrc;
    t.nK = p.K / KC;
    t.group_size = p.group_size;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int c = (tid + NT * i) % C::A_CHUNKS;
      const int r = c / (KC / 8), kc8 = c % (KC / 8);
      const int rr = row0 + min(r, rows - 1);
      int src = p.row_index ? p.row_index[rr] / p.row_div : rr;
      src = min(max(src, 0), p.a_rows - 1);
      // Rows past the tile's last row load through an offset beyond the descriptor's range: the
      // load returns zeros without a memory request (the host keeps a_rows * K * 2 below 2^31).
      t.a_off[i] = r < rows ? (uint32_t)(((size_t)src * p.K + kc8 * 8) * 2) : 0x80000000u;
    }
    // piece i of a thread lands SLICE_ROWS * i rows below piece 0 (the swizzle repeats every 16 rows)
    t.a_lds = lds_off_rows((tid % C::A_CHUNKS) / (KC / 8), tid % (KC / 8));
    if constexpr (C::KN) {
      // [K][N]: piece p of a matrix's chunk is row p / (BN / 8), 8 columns at chunk p % (BN / 8);
      // 16 (BN = 128) or 8 (BN = 64) lanes read one 256- or 128-byte row
      constexpr int per_m = KC * BN / 8;
      static_assert(per_m % 64 == 0, "a wave's pieces read one matrix");
#pragma unroll
      for (int m = 0; m < C::NW; ++m)
        t.wr[m] = make_rsrc(static_cast<const char*>(m == 0 ? p.w0 : p.w1) + (size_t)e * w_bytes, w_bytes);
#pragma unroll
      for (int x = 0; x < C::B_PIECES; ++x) {
        const int pidx = tid + NT * x;
        const int m = __builtin_amdgcn_readfirstlane(pidx / per_m);
        const int q = pidx % per_m, k = q / (BN / 8), c = q % (BN / 8);
        t.kn_m[x] = m;
        t.kn_voff[x] = (uint32_t)((k * p.N + c * 8) * 2);
        t.kn_dst[x] = m * BN * KC + k * BN + ((c ^ swz_kn<BN>(k)) << 3);
      }
      t.kn_soff = (uint32_t)n0 * 2;
      t.row_bytes = p.N * 2;
    } else if constexpr (C::W8) {
      // fp8 [e][n][k]
#pragma unroll
      for (int m = 0; m < C::NW; ++m)
        t.wr[m] = make_rsrc(static_cast<const char*>(m == 0 ? p.w0 : p.w1) + (size_t)e * w_bytes, w_bytes);
      t.w8_hi = false;
      if constexpr (C::W8PAIR) {
        // Pairs: piece x of a thread is piece Q = tid + NT x of the chunk pair, bytes 16 (Q % 8)
        // .. + 15 of the pair's 128 bytes of column Q / 8 (8 lanes read a whole line); a piece
        // belongs to the pair's first or second chunk by (Q % 8) / 4 and fills LDS chunks 2 kq
        // and + 1 (kq = Q % 4) of its column: the 4 lanes of a group that store one chunk write
        // 4 slots of one row.
        // Piece q's columns are NT / 8 q .. + NT / 8 - 1 of the tile, a compile-time matrix and
        // first column (NT / 8 divides BN, a multiple of 16 rows: the same swizzle), so a lane
        // keeps one global offset and one LDS destination per chunk half.
        static_assert(NT / 8 <= BN && BN % (NT / 8) == 0 && (NT / 8) % 16 == 0, "piece columns");
        t.w8_hi = ((lane & 7) >> 2) != 0;
        t.row_bytes = p.K;
        t.w8_off[0] = (uint32_t)((n0 + tid / 8) * p.K + (lane & 7) * 16);
#pragma unroll
        for (int c = 0; c < 2; ++c) t.b_dst[0][c] = lds_off_rows(tid / 8, 2 * (lane & 3) + c);
      } else {
        // Piece x of a thread is piece P = tid + NT x of the chunk, 16 consecutive k (bytes
        // 16 (P % 4) .. + 15) of column (P / 4) % BN of matrix P / (4 BN): four lanes read one
        // column's 64 bytes, so each load of a wave covers 16 whole 64-byte column segments.  A
        // piece fills LDS chunks 2 (P % 4) and + 1 of its column.  (16-byte LDS stores go 8 lanes
        // at a time through 32 banks, so the two columns of an 8-lane group collide once; dealing
        // columns two apart to a group avoids that but measured 4 % slower on the prefill tiles.)
        constexpr int per_m = KC * BN / 16;
        static_assert(per_m % 64 == 0, "a wave's pieces read one matrix");
#pragma unroll
        for (int x = 0; x < 2 * C::B_UNITS; ++x) {
          const int P = tid + NT * x;
          const int m = __builtin_amdgcn_readfirstlane(P / per_m);
          const int n = (P / 4) % BN, kq = P % 4;
          t.w8_m[x] = m;
          t.w8_off[x] = (uint32_t)((n0 + n) * p.K + kq * 16);
#pragma unroll
          for (int c = 0; c < 2; ++c) t.b_dst[x / 2][2 * (x % 2) + c] = lds_off_rows(m * BN + n, 2 * kq + c);
        }
      }
#pragma unroll
      for (int m = 0; m < C::NW; ++m)
        t.es[m] = static_cast<const u16*>(m == 0 ? p.s0 : p.s1) + (size_t)e * p.N + n0;
    } else if constexpr (!C::Q4) {
      // Weight rows are K-contiguous ([e][n][k]) and go to LDS like activation rows: 8 lanes per
      // 128-byte row chunk, wave w's lanes on rows 8w .. 8w+7 of every slice of SLICE_ROWS rows.
#pragma unroll
      for (int m = 0; m < C::NW; ++m)
        t.wr[m] = make_rsrc(static_cast<const char*>(m == 0 ? p.w0 : p.w1) + (size_t)e * w_bytes, w_bytes);
      t.row_bytes = p.K * 2;
      t.b_voff = (uint32_t)((lane >> 3) * t.row_bytes + (lane & 7) * 16);
      t.b_soff = (uint32_t)((n0 + wave * 8) * t.row_bytes);
      t.b_lds = lds_off_rows(wave * 8 + (lane >> 3), lane & 7);
    } else {
      // Unit i of a thread (one 16-byte row piece: 4 words of 8 k each, columns 4 nq .. 4 nq + 3 of
      // word row kw) reads matrix (tid + NT*i) / per_m, the same for the whole wave.  Within a
      // matrix, unit u covers kw = u % 8 and nq = u / 8: the 16 lanes of an LDS pass hold 8 word
      // rows of 2 adjacent column quads (nq even, nq odd), and a wave's loads are 8 whole 128-byte
      // rows.  Odd quads write their columns in the order 1, 0, 3, 2, so at every store the two
      // halves of a pass write rows of opposite parity: 8 chunks of an even row and 8 of an odd
      // row, one per bank group.
      constexpr int per_m = KC * BN / 32;
      static_assert(per_m % 64 == 0, "a wave's units read one matrix");
#pragma unroll
      for (int i = 0; i < C::B_UNITS; ++i) {
        const int m = __builtin_amdgcn_readfirstlane((tid + NT * i) / per_m);
        t.wr[i] = make_rsrc(static_cast<const char*>(m == 0 ? p.w0 : p.w1) + (size_t)e * w_bytes, w_bytes);
        t.sr[i] = make_rsrc(static_cast<const char*>(m == 0 ? p.s0 : p.s1) + (size_t)e * s_bytes, s_bytes);
      }
      t.row_bytes = p.N * 4;
      t.s_row_bytes = p.N * 2;
#pragma unroll
      for (int i = 0; i < C::B_UNITS; ++i) {
        const int u = (tid + NT * i) % per_m;
        const int kw = u % (KC / 8), nq = u / (KC / 8);
        const int m = (tid + NT * i) / per_m;
        const int sw = nq & 1;
        t.b_off[i] = (uint32_t)(kw * p.N + n0 + nq * 4) * 4u;
        // scale row of the word row's group inside a chunk (group sizes below 64)
        const int kg = p.group_size < KC ? kw * 8 / p.group_size : 0;
        t.s_off[i] = (uint32_t)(kg * p.N + n0 + nq * 4) * 2u;
        t.b_swap[i] = sw != 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) t.b_dst[i][c] = lds_off_rows(m * BN + nq * 4 + (c ^ sw), kw);
      }
    }
    tile_dispatch<C, OutT, 0>(nm, t, buf0, buf1, O, p.N, lane, wrow0, wcol0, row0, rows, n0, p.bias);
  }
}

// ---------------------------------------------------------------------------------------------
// One-buffer tiles, dense weights, activation rows in sorted order (no gather): chunk loads run
// across tile boundaries.  A workgroup that owns several tiles (the down projection of a
// decode-shaped batch: K = I is short, N = H wide) loads the first two chunks of its next tile
// behind the last two chunks of the current one, so they are in flight during that tile's last
// MFMAs and its epilogue.  Same tiles, LDS layout, operand reads and epilogue as k_gemm_bf16.
// ---------------------------------------------------------------------------------------------
// Loading context of one tile; valid = false gives descriptors of range 0 (every load returns
// zeros without a memory request).
template <class C>
__device__ __forceinline__ TileCtx<C> stream_ctx(const GemmParams& p, const TileCoord& tc, bool valid, uint32_t a_bytes,
                                                 uint32_t w_bytes, int tid, int lane, int wave) {
  TileCtx<C> t;
  t.ar = make_rsrc(p.a, valid ? a_bytes : 0u);
  t.nK = p.K / C::KC;
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int c = (tid + C::NT * i) % C::A_CHUNKS;
    const int r = c / (C::KC / 8), kc8 = c % (C::KC / 8);
    const int src = min(tc.row0 + min(r, tc.rows - 1), p.a_rows - 1);
    t.a_off[i] = r < tc.rows ? (uint32_t)(((size_t)src * p.K + kc8 * 8) * 2) : 0x80000000u;
  }
  t.a_lds = lds_off_rows((tid % C::A_CHUNKS) / (C::KC / 8), tid % (C::KC / 8));
#pragma unroll
  for (int m = 0; m < C::NW; ++m)
    t.wr[m] = make_rsrc(static_cast<const char*>(m == 0 ? p.w0 : p.w1) + (size_t)tc.e * w_bytes, valid ? w_bytes : 0u);
  t.row_bytes = p.K * 2;
  t.b_voff = (uint32_t)((lane >> 3) * t.row_bytes + (lane & 7) * 16);
  t.b_soff = (uint32_t)((tc.n0 + wave * 8) * t.row_bytes);
  t.b_lds = lds_off_rows(wave * 8 + (lane >> 3), lane & 7);
  return t;
}

// Epilogue: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16 tile (SwiGLU of the gate
// and up values for gate/up tiles); rows past the tile's last row are not written.
template <class C, typename OutT, int NM, int NA = (NM > 0 ? NM : 1)>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[C::NW][NA][C::NTL], OutT* O, int N, int lane,
                                           int wrow0, int wcol0, int row0, int rows, int n0) {
#pragma unroll
  for (int i = 0; i < NM; ++i)
#pragma unroll
    for (int j = 0; j < C::NTL; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wrow0 + i * 16 * C::WM + (lane >> 4) * 4 + r;
        const int col = wcol0 + j * 16 + (lane & 15);
        if (row < rows) {
          float v;
          if constexpr (C::GU) v = silu_mul(acc[0][i][j][r] * C::OUT_MUL, acc[1][i][j][r] * C::OUT_MUL);
          else v = acc[0][i][j][r] * C::OUT_MUL;
          store_out(O + (size_t)(row0 + row) * N + n0 + col, v);
        }
      }
}

// MFMAs of one LDS chunk, or the epilogue, for nm (wave-uniform) live 16-row tiles on accumulators
// sized for the largest count: only a branch picks the instance, so the registers of the chunks
// in flight stay where they are.
template <class C, int NM = 1>
__device__ __forceinline__ void compute_chunk_nm(int nm, const u16* buf, f32x4 (&acc)[C::NW][C::MT][C::NTL],
                                                 int arow, int bcol, int kofs) {
  if constexpr (NM <= C::MT) {
    if (nm == NM) compute_chunk<C, NM, C::MT>(buf, acc, arow, bcol, kofs);
    else compute_chunk_nm<C, NM + 1>(nm, buf, acc, arow, bcol, kofs);
  }
}
template <class C, typename OutT, int NM = 1>
__device__ __forceinline__ void store_tile_nm(int nm, const f32x4 (&acc)[C::NW][C::MT][C::NTL], OutT* O, int N,
                                              int lane, int wrow0, int wcol0, const TileCoord& tc) {
  if constexpr (NM <= C::MT) {
    if (nm == NM) store_tile<C, OutT, NM, C::MT>(acc, O, N, lane, wrow0, wcol0, tc.row0, tc.rows, tc.n0);
    else store_tile_nm<C, OutT, NM + 1>(nm, acc, O, N, lane, wrow0, wcol0, tc);
  }
}

template <class C, typename OutT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_SIMD)))
void k_gemm_stream(GemmParams p) {
  static_assert(C::STAGES == 1 && !C::Q4, "one LDS buffer, dense weights");
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN;
  extern __shared__ __attribute__((aligned(16))) u16 smem[];
  u16* buf = smem;
  int* s_tstart = reinterpret_cast<int*>(smem + C::STAGE);
  int* s_goff = s_tstart + (p.n_groups + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = p.N / BN;
  const int wrow0 = wm * 16, wcol0 = wn * (BN / WN);
  build_tile_table(p, BM, tiles_n, s_tstart, s_goff);
  __syncthreads();
  const TileIter it = tile_range(s_tstart[p.n_groups]);
  if (it.next >= it.end) return;
  OutT* O = static_cast<OutT*>(p.out);
  // the host checks a_rows * K * 2 < 2^31 and K * N * 2 < 2^32
  const uint32_t a_bytes = (uint32_t)((size_t)p.a_rows * p.K * 2), w_bytes = (uint32_t)((size_t)p.K * p.N * 2);
  const int arow = wrow0 + (lane & 15), bcol = wcol0 + (lane & 15), kofs = (lane >> 4) * 8;

  TileCoord tc = tile_coord(s_tstart, s_goff, p.n_groups, it.next, BM, BN, tiles_n);
  TileCtx<C> t = stream_ctx<C>(p, tc, true, a_bytes, w_bytes, tid, lane, wave);
  Chunk<C> c0, c1;
  load_chunk(t, 0, c0);
  load_chunk(t, 1, c1);
  for (int tile = it.next; tile < it.end; tile += it.step) {
    const bool more = tile + it.step < it.end;        // after the last tile: loads of range 0
    const TileCoord tcn = tile_coord(s_tstart, s_goff, p.n_groups, more ? tile + it.step : tile, BM, BN, tiles_n);
    const TileCtx<C> tn = stream_ctx<C>(p, tcn, more, a_bytes, w_bytes, tid, lane, wave);
    const int nm = min(C::MT, max(0, ((tc.rows + 15) / 16 - wm + WM - 1) / WM));   // live 16-row tiles
    f32x4 acc[C::NW][C::MT][C::NTL];
#pragma unroll
    for (int m = 0; m < C::NW; ++m)
#pragma unroll
      for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int j = 0; j < C::NTL; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the chunk count is even: chunks kc and kc + 1 sit in c0 and c1
    for (int kc = 0; kc + 2 < t.nK; kc += 2) {
      store_chunk(t, c0, buf);
      __syncthreads();
      compute_chunk_nm<C>(nm, buf, acc, arow, bcol, kofs);
      load_chunk(t, kc + 2, c0);
      __syncthreads();
      store_chunk(t, c1, buf);
      __syncthreads();
      compute_chunk_nm<C>(nm, buf, acc, arow, bcol, kofs);
      load_chunk(t, kc + 3, c1);
      __syncthreads();
    }
    store_chunk(t, c0, buf);
    __syncthreads();
    compute_chunk_nm<C>(nm, buf, acc, arow, bcol, kofs);
    load_chunk(tn, 0, c0);
    __syncthreads();
    store_chunk(t, c1, buf);
    __syncthreads();
    compute_chunk_nm<C>(nm, buf, acc, arow, bcol, kofs);
    load_chunk(tn, 1, c1);
    __syncthreads();                               // LDS is refilled by the next tile
    store_tile_nm<C, OutT>(nm, acc, O, p.N, lane, wrow0, wcol0, tc);
    tc = tcn;
    t = tn;
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 MFMA kernel with direct global -> LDS loads (dense weights, prefill tiles)
// ---------------------------------------------------------------------------------------------
// Same tiles, LDS layout, operand reads and epilogue as k_gemm_bf16, but activation rows and
// weight rows go from global memory straight into LDS (buffer_load_dwordx4 ... lds): no staging
// registers, no ds_write instructions, so more of the issue slots and registers stay with the
// MFMA stream.  One load instruction fills 8 consecutive 128-byte rows (lane i writes the 16 bytes
// at M0 + 16 i), so the row swizzle is applied on the global side: lane i loads the chunk that
// belongs at position i % 8 of row i / 8.  Two LDS buffers: while chunk kc is multiplied from one,
// chunk kc + 1 streams into the other.
//
// The loads are issued from inline assembly, which the compiler's wait-count tracking does not
// see (with the compiler's own LDS-load intrinsic it waits for every outstanding load before each
// LDS read, which serialises the pipeline): the kernel waits for them itself (s_waitcnt vmcnt(0)
// before the barrier that publishes a buffer; vector memory operations of a wave complete in
// issue order, and any other outstanding vector memory operation only makes the wait longer).
// F16_: fp16 operands (activations already fp16, weights carrying 2^8), else bf16.
template <int BM_, int BN_, int WM_, int WN_, bool GU_, bool F16_ = false>
struct DCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool GU = GU_, F16 = F16_;
  static constexpr float OUT_MUL = F16_ ? 1.0f / kF16WeightScale : 1.0f;
  static constexpr int NWAVES = WM * WN, NT = 64 * NWAVES;
  static constexpr int WAVES_PER_SIMD = (NWAVES + 3) / 4;
  static constexpr int KC = 64, NW = GU ? 2 : 1;
  static constexpr int A_ELEMS = BM * 64, B_ELEMS = NW * BN * 64, STAGE = A_ELEMS + B_ELEMS;
  static constexpr int A_INST = BM / 8 / NWAVES, B_INST = NW * BN / 8 / NWAVES;
  static constexpr int MT = BM / WM / 16, NTL = BN / WN / 16;
  static_assert(A_INST >= 1 && B_INST >= 1 && BM % (8 * NWAVES) == 0 && BN % 8 == 0, "row blocks");
  static_assert(NWAVES % 2 == 0, "8-row block parity equals the wave's parity (global-side swizzle)");
  static size_t lds_bytes(int n_groups) { return 2 * (size_t)STAGE * 2 + 2 * sizeof(int) * (n_groups + 1) + 16; }
};

// One 16-byte-per-lane load into LDS: lane i's data lands at lds + 16 i (lds wave-uniform).  M0 is
// not used by anything else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"      // m0 is a reserved register; listing it is deliberate
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector memory instructions of this wave are outstanding (they complete in
// issue order, so every older one has landed).
template <int N>
__device__ __forceinline__ void wait_vmcnt_n() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

template <class C>
struct DmaCtx {
  __amdgpu_buffer_rsrc_t ar, wr[C::NW];             // activation matrix; the tile's expert weights
  uint32_t a_voff[C::A_INST];                       // lane's activation row piece per block (rows past the tile: out of range)
  uint32_t b_voff;                                  // lane's offset inside an 8-row weight block
  uint32_t b_soff[C::B_INST];                       // wave-uniform offset of each weight block
  int b_m[C::B_INST];                               // matrix of each weight block
  uint32_t lds;                                     // LDS address of buffer 0
  int wave, nK;
};

template <class C>
__device__ __forceinline__ void dma_chunk(const DmaCtx<C>& t, int kc, int stage) {
  const uint32_t st = t.lds + (uint32_t)stage * C::STAGE * 2;
  const uint32_t koff = (uint32_t)kc * 128;
#pragma unroll
  for (int j = 0; j < C::A_INST; ++j) lds_dma16(t.ar, t.a_voff[j], koff, st + 8 * (t.wave + C::NWAVES * j) * 128);
#pragma unroll
  for (int j = 0; j < C::B_INST; ++j) {
    __amdgpu_buffer_rsrc_t w = t.wr[0];
    if constexpr (C::NW == 2) w = t.b_m[j] ? t.wr[1] : t.wr[0];
    lds_dma16(w, t.b_voff, t.b_soff[j] + koff, st + C::A_ELEMS * 2 + 8 * (t.wave + C::NWAVES * j) * 128);
  }
}

template <class C>
__device__ __forceinline__ void dma_a(const DmaCtx<C>& t, int kc, int stage) {
  const uint32_t st = t.lds + (uint32_t)stage * C::STAGE * 2;
#pragma unroll
  for (int j = 0; j < C::A_INST; ++j)
    lds_dma16(t.ar, t.a_voff[j], (uint32_t)kc * 128, st + 8 * (t.wave + C::NWAVES * j) * 128);
}

// BREG: the tile's weight chunks go through registers two chunks ahead (global loads, then
// ds_write to where the copies would land), its activation chunks are copied one chunk ahead.
// For gate/up tiles whose expert has a single m-tile, whose weights therefore stream from HBM
// once: the register path gives their misses two chunks of time (prefill gate/up -4 %); tiles of
// experts with several m-tiles, whose weights the m-tiles share in L2, keep the copies (there the
// register path measured 6 % slower).
template <class C, typename OutT, int NM, bool BREG>
__device__ __forceinline__ void dma_tile(const DmaCtx<C>& t, u16* smem, OutT* O, int N, int lane, int wrow0, int wcol0,
                                         const TileCoord& tc) {
  f32x4 acc[C::NW][NM > 0 ? NM : 1][C::NTL];
#pragma unroll
  for (int m = 0; m < C::NW; ++m)
#pragma unroll
    for (int i = 0; i < (NM > 0 ? NM : 1); ++i)
#pragma unroll
      for (int j = 0; j < C::NTL; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int arow = wrow0 + (lane & 15), bcol = wcol0 + (lane & 15), kofs = (lane >> 4) * 8;
  const int nK = t.nK;
  // weights through registers: chunk kc + 1's weights are stored to LDS and chunk kc + 2's loaded
  // at the top of step kc; the loads land where the copies would (same lanes, same offsets)
  u32x4 wb[BREG ? C::B_INST : 1];
  auto wload = [&](int kc) {
    if constexpr (BREG) {
      kc = min(kc, nK - 1);
#pragma unroll
      for (int j = 0; j < C::B_INST; ++j) {
        __amdgpu_buffer_rsrc_t w = t.wr[0];
        if constexpr (C::NW == 2) w = t.b_m[j] ? t.wr[1] : t.wr[0];
        wb[j] = __builtin_amdgcn_raw_buffer_load_b128(w, t.b_voff, t.b_soff[j] + (uint32_t)kc * 128, 0);
      }
    }
  };
  auto wstore = [&](int stage) {
    if constexpr (BREG) {
      u16* sB = smem + stage * C::STAGE + C::A_ELEMS;
#pragma unroll
      for (int j = 0; j < C::B_INST; ++j)
        *reinterpret_cast<u32x4*>(sB + 8 * (t.wave + C::NWAVES * j) * 64 + lane * 8) = wb[j];
    }
  };
  wait_vmcnt0();
  if constexpr (BREG) {
    wload(0);
    wstore(0);
    dma_a(t, 0, 0);
    wload(1);
  } else {
    dma_chunk(t, 0, 0);
  }
  for (int kc = 0; kc < nK; ++kc) {
    if constexpr (BREG) wait_vmcnt_n<C::B_INST>();   // this wave's copies of chunk kc (weights of kc + 1 fly)
    else wait_vmcnt0();                                 // this wave's loads of chunk kc
    __syncthreads();                               // everyone's; and the other buffer is free
    if constexpr (BREG) {
      if (kc + 1 < nK) {
        wstore((kc + 1) & 1);
        dma_a(t, kc + 1, (kc + 1) & 1);
      }
      wload(kc + 2);                               // clamped past the end
    } else {
      if (kc + 1 < nK) dma_chunk(t, kc + 1, (kc + 1) & 1);
    }
    if constexpr (NM > 0) {
      const u16* sA = smem + (kc & 1) * C::STAGE;
      const u16* sB = sA + C::A_ELEMS;
      // Every operand of the chunk is read before its MFMAs: LDS reads return in order, so each
      // MFMA waits only for its own operands and the later reads overlap the earlier MFMAs.  With
      // weights in registers (16 more) one 32-k step's operands are read at a time.
      constexpr int KS = C::KC / 32;
      u32x4 av[KS][NM], bv[KS][C::NW][C::NTL];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (BREG) {
          if (ks > 0) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < C::NW; ++m)
#pragma unroll
              for (int j = 0; j < C::NTL; ++j)
#pragma unroll
                for (int i = 0; i < NM; ++i)
                  acc[m][i][j] = mma<C::F16>(av[ks - 1][i], bv[ks - 1][m][j], acc[m][i][j]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int i = 0; i < NM; ++i)
          av[ks][i] = *reinterpret_cast<const u32x4*>(sA + lds_off_rows(arow, (ks * 32 + kofs) >> 3) + i * 16 * C::WM * 64);
#pragma unroll
        for (int m = 0; m < C::NW; ++m)
#pragma unroll
          for (int j = 0; j < C::NTL; ++j)
            bv[ks][m][j] = *reinterpret_cast<const u32x4*>(sB + lds_off_rows(bcol, (ks * 32 + kofs) >> 3) + (m * C::BN + j * 16) * 64);
      }
      __builtin_amdgcn_sched_barrier(0);           // keep the reads ahead of the MFMAs
#pragma unroll
      for (int ks = BREG ? KS - 1 : 0; ks < KS; ++ks)
#pragma unroll
        for (int m = 0; m < C::NW; ++m)
#pragma unroll
          for (int j = 0; j < C::NTL; ++j)
#pragma unroll
            for (int i = 0; i < NM; ++i)
              acc[m][i][j] = mma<C::F16>(av[ks][i], bv[ks][m][j], acc[m][i][j]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NM; ++i)
#pragma unroll
    for (int j = 0; j < C::NTL; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wrow0 + i * 16 * C::WM + (lane >> 4) * 4 + r;
        const int col = wcol0 + j * 16 + (lane & 15);
        if (row < tc.rows) {
          float v;
          if constexpr (C::GU) v = silu_mul(acc[0][i][j][r] * C::OUT_MUL, acc[1][i][j][r] * C::OUT_MUL);
          else v = acc[0][i][j][r] * C::OUT_MUL;
          store_out(O + (size_t)(tc.row0 + row) * N + tc.n0 + col, v);
        }
      }
}

template <class C, typename OutT, int NM, bool BREG>
__device__ __forceinline__ void dma_dispatch(int nm, const DmaCtx<C>& t, u16* smem, OutT* O, int N, int lane, int wrow0,
                                             int wcol0, const TileCoord& tc) {
  if constexpr (NM <= C::MT) {
    if (nm == NM) dma_tile<C, OutT, NM, BREG>(t, smem, O, N, lane, wrow0, wcol0, tc);
    else dma_dispatch<C, OutT, NM + 1, BREG>(nm, t, smem, O, N, lane, wrow0, wcol0, tc);
  }
}

// GATHER: activation rows through row_index / row_div; false: row r of the tile reads row r of a
// (identity rows, e.g. the shared expert), with no index loads.
template <class C, typename OutT, bool GATHER>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_SIMD)))
void k_gemm_dma(GemmParams p) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN;
  extern __shared__ __attribute__((aligned(16))) u16 smem_dma[];
  int* s_tstart = reinterpret_cast<int*>(smem_dma + 2 * C::STAGE);
  int* s_goff = s_tstart + (p.n_groups + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = p.N / BN;
  const int wrow0 = wm * 16, wcol0 = wn * (BN / WN);
  build_tile_table(p, BM, tiles_n, s_tstart, s_goff);
  __syncthreads();
  const int total = s_tstart[p.n_groups];
  const TileIter it = tile_range(total);
  DmaCtx<C> t;
  t.ar = make_rsrc(p.a, (uint32_t)((size_t)p.a_rows * p.K * 2));
  t.wave = wave;
  t.nK = p.K / C::KC;
  t.lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)smem_dma);
  const uint32_t w_bytes = (uint32_t)((size_t)p.K * p.N * 2);
  const uint32_t row_bytes = (uint32_t)p.K * 2;
  // lane i fills row i / 8 of an 8-row block at chunk position i % 8; the block starts at a row
  // 8 * (wave + NWAVES * j), so the row's swizzle (row / 2) mod 8 is (i / 16) ^ 4 * (wave & 1)
  const int q = (lane & 7) ^ (lane >> 4) ^ (4 * (wave & 1));
  t.b_voff = (uint32_t)(lane >> 3) * row_bytes + q * 16;
  OutT* O = static_cast<OutT*>(p.out);
  for (int tile = it.next; tile < it.end; tile += it.step) {
    const TileCoord tc = tile_coord(s_tstart, s_goff, p.n_groups, tile, BM, BN, tiles_n);
    const int nm = min(C::MT, max(0, ((tc.rows + 15) / 16 - wm + WM - 1) / WM));
#pragma unroll
    for (int m = 0; m < C::NW; ++m)
      t.wr[m] = make_rsrc(static_cast<const char*>(m == 0 ? p.w0 : p.w1) + (size_t)tc.e * w_bytes, w_bytes);
#pragma unroll
    for (int j = 0; j < C::A_INST; ++j) {
      const int r = 8 * (wave + C::NWAVES * j) + (lane >> 3);
      const int rr = tc.row0 + min(r, tc.rows - 1);
      int src = GATHER ? p.row_index[rr] / p.row_div : rr;
      src = min(max(src, 0), p.a_rows - 1);
      t.a_voff[j] = r < tc.rows ? (uint32_t)(((size_t)src * p.K + q * 8) * 2) : 0x80000000u;
    }
#pragma unroll
    for (int j = 0; j < C::B_INST; ++j) {
      const int rb = 8 * (wave + C::NWAVES * j);
      t.b_m[j] = rb / BN;
      t.b_soff[j] = (uint32_t)(tc.n0 + rb % BN) * row_bytes;
    }
    // gate/up tiles of an expert with one m-tile: its weights stream once, through registers
    const bool once = C::GU && __builtin_amdgcn_readfirstlane(s_goff[tc.e + 1] - s_goff[tc.e]) <= BM;
    if constexpr (C::GU) {
      if (once) {
        dma_dispatch<C, OutT, 0, true>(nm, t, smem_dma, O, p.N, lane, wrow0, wcol0, tc);
        continue;
      }
    }
    dma_dispatch<C, OutT, 0, false>(nm, t, smem_dma, O, p.N, lane, wrow0, wcol0, tc);
  }
}

// ---------------------------------------------------------------------------------------------
// The same tiles with three weight buffers: weight chunks are copied two chunks ahead (activation
// chunks, mostly L2 hits, one ahead).  Two activation and three weight buffers of a 256-row tile
// take all 160 KB of LDS, so the tile table lives in registers instead (one lane per expert, up
// to 64 experts): every wave scans the group sizes itself and finds a tile's expert with a ballot.
// ---------------------------------------------------------------------------------------------
struct RegTable {
  int lo, hi, tstart;                              // lane e: rows [lo, hi) of group e, its first tile
  int total;
};

__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return x;
}

// Same tile numbering as build_tile_table (n_groups <= 64).
__device__ __forceinline__ RegTable reg_tile_table(const GemmParams& p, int BM, int tiles_n, int lane) {
  RegTable r;
  int tiles = 0;
  r.lo = 0;
  r.hi = 0;
  if (lane < p.n_groups) {
    r.lo = min(max(p.group_offsets ? p.group_offsets[lane] : 0, 0), p.rows_cap);
    r.hi = min(max(p.group_offsets ? p.group_offsets[lane + 1] : p.rows_cap, r.lo), p.rows_cap);
    tiles = ((r.hi - r.lo + BM - 1) / BM) * tiles_n;
  }
  const int incl = wave_scan_incl(tiles);
  r.tstart = incl - tiles;
  r.total = __builtin_amdgcn_readlane(incl, 63);
  return r;
}

__device__ __forceinline__ TileCoord reg_tile_coord(const RegTable& r, int n_groups, int lane, int tile, int BM, int BN,
                                                    int tiles_n) {
  constexpr int kGroupM = 4;
  // the expert is the last group whose first tile is <= tile (empty groups before it start at or
  // before it, those after it start after it)
  const uint64_t m = __ballot(lane < n_groups && r.tstart <= tile);
  const int e = 63 - __builtin_clzll(m);
  const int g0 = __builtin_amdgcn_readlane(r.lo, e), g1 = __builtin_amdgcn_readlane(r.hi, e);
  const int local = tile - __builtin_amdgcn_readlane(r.tstart, e);
  const int mtiles = (g1 - g0 + BM - 1) / BM;
  const int grp = local / (kGroupM * tiles_n), in_grp = local % (kGroupM * tiles_n);
  const int gm = min(kGroupM, mtiles - grp * kGroupM);
  const int mt = grp * kGroupM + in_grp % gm, nt = in_grp / gm;
  const int row0 = g0 + mt * BM;
  return {e, row0, min(BM, g1 - row0), nt * BN};
}


// LDS: activation buffers [2][A_ELEMS], then weight buffers [3][B_ELEMS].
template <class C>
__device__ __forceinline__ void dma3_a(const DmaCtx<C>& t, int kc, int buf) {
  const uint32_t st = t.lds + (uint32_t)buf * C::A_ELEMS * 2;
#pragma unroll
  for (int j = 0; j < C::A_INST; ++j)
    lds_dma16(t.ar, t.a_voff[j], (uint32_t)kc * 128, st + 8 * (t.wave + C::NWAVES * j) * 128);
}
template <class C>
__device__ __forceinline__ void dma3_b(const DmaCtx<C>& t, int kc, int buf) {
  const uint32_t st = t.lds + (uint32_t)(2 * C::A_ELEMS + buf * C::B_ELEMS) * 2;
#pragma unroll
  for (int j = 0; j < C::B_INST; ++j) {
    __amdgpu_buffer_rsrc_t w = t.wr[0];
    if constexpr (C::NW == 2) w = t.b_m[j] ? t.wr[1] : t.wr[0];
    lds_dma16(w, t.b_voff, t.b_soff[j] + (uint32_t)kc * 128, st + 8 * (t.wave + C::NWAVES * j) * 128);
  }
}

template <class C, typename OutT, int NM>
__device__ __forceinline__ void dma3_tile(const DmaCtx<C>& t, u16* smem, OutT* O, int N, int lane, int wrow0, int wcol0,
                                          const TileCoord& tc) {
  f32x4 acc[C::NW][NM > 0 ? NM : 1][C::NTL];
#pragma unroll
  for (int m = 0; m < C::NW; ++m)
#pragma unroll
    for (int i = 0; i < (NM > 0 ? NM : 1); ++i)
#pragma unroll
      for (int j = 0; j < C::NTL; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int arow = wrow0 + (lane & 15), bcol = wcol0 + (lane & 15), kofs = (lane >> 4) * 8;
  const int nK = t.nK;
  // Issue order: A(0), B(0), B(1); iteration kc then issues A(kc+1) and B(kc+2).  At the top of
  // iteration kc only weight chunk kc+1 may still be outstanding after A(kc) and B(kc).
  wait_vmcnt0();                                   // nothing of the previous tile is in flight
  dma3_a(t, 0, 0);
  dma3_b(t, 0, 0);
  if (nK > 1) dma3_b(t, 1, 1);
  int sb = 0;                                      // weight buffer of chunk kc
  for (int kc = 0; kc < nK; ++kc) {
    if (kc + 1 < nK) wait_vmcnt_n<C::B_INST>();
    else wait_vmcnt0();
    __syncthreads();                               // everyone's chunk kc; buffers of chunk kc-1 free
    if (kc + 1 < nK) dma3_a(t, kc + 1, (kc + 1) & 1);
    if (kc + 2 < nK) dma3_b(t, kc + 2, sb == 0 ? 2 : sb - 1);
    if constexpr (NM > 0) {
      const u16* sA = smem + (kc & 1) * C::A_ELEMS;
      const u16* sB = smem + 2 * C::A_ELEMS + sb * C::B_ELEMS;
      constexpr int KS = C::KC / 32;
      u32x4 av[KS][NM], bv[KS][C::NW][C::NTL];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < NM; ++i)
          av[ks][i] = *reinterpret_cast<const u32x4*>(sA + lds_off_rows(arow, (ks * 32 + kofs) >> 3) + i * 16 * C::WM * 64);
#pragma unroll
        for (int m = 0; m < C::NW; ++m)
#pragma unroll
          for (int j = 0; j < C::NTL; ++j)
            bv[ks][m][j] = *reinterpret_cast<const u32x4*>(sB + lds_off_rows(bcol, (ks * 32 + kofs) >> 3) + (m * C::BN + j * 16) * 64);
      }
      __builtin_amdgcn_sched_barrier(0);           // keep the reads ahead of the MFMAs
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int m = 0; m < C::NW; ++m)
#pragma unroll
          for (int j = 0; j < C::NTL; ++j)
#pragma unroll
            for (int i = 0; i < NM; ++i)
              acc[m][i][j] = mma<C::F16>(av[ks][i], bv[ks][m][j], acc[m][i][j]);
    }
    sb = sb == 2 ? 0 : sb + 1;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NM; ++i)
#pragma unroll
    for (int j = 0; j < C::NTL; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wrow0 + i * 16 * C::WM + (lane >> 4) * 4 + r;
        const int col = wcol0 + j * 16 + (lane & 15);
        if (row < tc.rows) {
          float v;
          if constexpr (C::GU) v = silu_mul(acc[0][i][j][r] * C::OUT_MUL, acc[1][i][j][r] * C::OUT_MUL);
          else v = acc[0][i][j][r] * C::OUT_MUL;
          store_out(O + (size_t)(tc.row0 + row) * N + tc.n0 + col, v);
        }
      }
}

template <class C, typename OutT, int NM>
__device__ __forceinline__ void dma3_dispatch(int nm, const DmaCtx<C>& t, u16* smem, OutT* O, int N, int lane,
                                              int wrow0, int wcol0, const TileCoord& tc) {
  if constexpr (NM <= C::MT) {
    if (nm == NM) dma3_tile<C, OutT, NM>(t, smem, O, N, lane, wrow0, wcol0, tc);
    else dma3_dispatch<C, OutT, NM + 1>(nm, t, smem, O, N, lane, wrow0, wcol0, tc);
  }
}

template <class C, typename OutT>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_SIMD)))
void k_gemm_dma3(GemmParams p) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN;
  extern __shared__ __attribute__((aligned(16))) u16 smem_dma3[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = p.N / BN;
  const int wrow0 = wm * 16, wcol0 = wn * (BN / WN);
  const RegTable tab = reg_tile_table(p, BM, tiles_n, lane);
  const TileIter it = tile_range(tab.total);
  DmaCtx<C> t;
  t.ar = make_rsrc(p.a, (uint32_t)((size_t)p.a_rows * p.K * 2));
  t.wave = wave;
  t.nK = p.K / C::KC;
  t.lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)smem_dma3);
  const uint32_t w_bytes = (uint32_t)((size_t)p.K * p.N * 2);
  const uint32_t row_bytes = (uint32_t)p.K * 2;
  // lane i fills row i / 8 of an 8-row block at chunk position i % 8; the block starts at a row
  // 8 * (wave + NWAVES * j), so the row's swizzle (row / 2) mod 8 is (i / 16) ^ 4 * (wave & 1)
  const int q = (lane & 7) ^ (lane >> 4) ^ (4 * (wave & 1));
  t.b_voff = (uint32_t)(lane >> 3) * row_bytes + q * 16;
  OutT* O = static_cast<OutT*>(p.out);
  for (int tile = it.next; tile < it.end; tile += it.step) {
    const TileCoord tc = reg_tile_coord(tab, p.n_groups, lane, tile, BM, BN, tiles_n);
    const int nm = min(C::MT, max(0, ((tc.rows + 15) / 16 - wm + WM - 1) / WM));
#pragma unroll
    for (int m = 0; m < C::NW; ++m)
      t.wr[m] = make_rsrc(static_cast<const char*>(m == 0 ? p.w0 : p.w1) + (size_t)tc.e * w_bytes, w_bytes);
#pragma unroll
    for (int j = 0; j < C::A_INST; ++j) {
      const int r = 8 * (wave + C::NWAVES * j) + (lane >> 3);
      const int rr = tc.row0 + min(r, tc.rows - 1);
      int src = p.row_index ? p.row_index[rr] / p.row_div : rr;
      src = min(max(src, 0), p.a_rows - 1);
      t.a_voff[j] = r < tc.rows ? (uint32_t)(((size_t)src * p.K + q * 8) * 2) : 0x80000000u;
    }
#pragma unroll
    for (int j = 0; j < C::B_INST; ++j) {
      const int rb = 8 * (wave + C::NWAVES * j);
      t.b_m[j] = rb / BN;
      t.b_soff[j] = (uint32_t)(tc.n0 + rb % BN) * row_bytes;
    }
    dma3_dispatch<C, OutT, 0>(nm, t, smem_dma3, O, p.N, lane, wrow0, wcol0, tc);
  }
}

// Launchers.  Each is called only for a shape it handles (the caller checks N against the tile
// width and the LDS sizes first), so any error they return is a real launch failure.
template <class C, typename OutT>
hipError_t run_dma3(const GemmParams& p, hipStream_t s) {
  static_assert((size_t)(2 * C::A_ELEMS + 3 * C::B_ELEMS) * 2 <= kLdsPerCu, "three weight buffers fit in LDS");
  const size_t lds = (size_t)(2 * C::A_ELEMS + 3 * C::B_ELEMS) * 2;
  const long long max_tiles = ((long long)(p.rows_cap + C::BM - 1) / C::BM + p.n_groups) * (p.N / C::BN);
  long long grid = device_cu_count();
  if (grid > max_tiles) grid = max_tiles;
  grid = ((grid + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  k_gemm_dma3<C, OutT><<<dim3((unsigned)grid), dim3(C::NT), lds, s>>>(p);
  return hipGetLastError();
}

template <class C, typename OutT>
hipError_t run_dma(const GemmParams& p, hipStream_t s) {
  static_assert(2 * (size_t)C::STAGE * 2 + 2 * 4 * 1025 + 16 <= kLdsPerCu, "two buffers and a 1024-group tile table fit in LDS");
  const size_t lds = C::lds_bytes(p.n_groups);
  const long long max_tiles = ((long long)(p.rows_cap + C::BM - 1) / C::BM + p.n_groups) * (p.N / C::BN);
  long long grid = device_cu_count();
  if (grid > max_tiles) grid = max_tiles;
  grid = ((grid + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  if (p.row_index)
    k_gemm_dma<C, OutT, true><<<dim3((unsigned)grid), dim3(C::NT), lds, s>>>(p);
  else
    k_gemm_dma<C, OutT, false><<<dim3((unsigned)grid), dim3(C::NT), lds, s>>>(p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// fp32 kernel: 32 x 64 tiles, K chunks of 32 staged in LDS, fp32 MFMA (16x16x4) with fp32 accumulation.
// ---------------------------------------------------------------------------------------------
// NK: weights stored [e][n][k] (MOE_W_DENSE_NK), else [e][k][n] (MOE_W_DENSE).
template <bool GU, bool NK>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmParams p) {
  constexpr int BM = 32, BN = 64, KC = 32, NW = GU ? 2 : 1;
  __shared__ float sA[BM][KC + 1];
  __shared__ float sB[NW][BN][KC + 1];             // weight rows [n][k], padded
  extern __shared__ int tbl[];
  int* s_tstart = tbl;
  int* s_goff = tbl + (p.n_groups + 1);
  // MFMA 16x16x4 fp32: wave w computes output columns 16 w .. 16 w + 15 of both 16-row blocks;
  // lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] of each 4-k step and holds rows
  // 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16 of the result
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int tiles_n = p.N / BN;
  build_tile_table(p, BM, tiles_n, s_tstart, s_goff);
  __syncthreads();
  const int total = s_tstart[p.n_groups];
  const TileIter it = tile_range(total);
  const float* A = static_cast<const float*>(p.a);
  float* O = static_cast<float*>(p.out);

  for (int tile = it.next; tile < it.end; tile += it.step) {
    const int e = find_group(s_tstart, p.n_groups, tile);
    const int g0 = s_goff[e], g1 = s_goff[e + 1];
    const int mtiles = (g1 - g0 + BM - 1) / BM;
    const int local = tile - s_tstart[e];
    const int mt = local % mtiles, nt = local / mtiles;
    const int row0 = g0 + mt * BM, rows = min(BM, g1 - row0), n0 = nt * BN;
    f32x4 acc[NW][2];
#pragma unroll
    for (int m = 0; m < NW; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // source rows of this thread's activation elements (fixed for the tile)
    constexpr int A_PER = BM * KC / 256, B_PER = NW * KC * BN / 256;
    const float* a_src[A_PER];
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
      const int r = (tid + 256 * u) / KC;
      const int rr = row0 + min(r, rows - 1);
      int src = p.row_index ? p.row_index[rr] / p.row_div : rr;
      src = min(max(src, 0), p.a_rows - 1);
      a_src[u] = A + (size_t)src * p.K + (tid + 256 * u) % KC;
    }
    // chunk loads (consecutive threads read contiguous memory); the next chunk's are issued
    // before the current chunk's products, so their latency overlaps them
    float av[A_PER], bv[B_PER];
    auto load = [&](int k0) {
#pragma unroll
      for (int u = 0; u < A_PER; ++u) av[u] = a_src[u][k0];
#pragma unroll
      for (int u = 0; u < B_PER; ++u) {
        const int i = tid + 256 * u;
        const int m = i / (KC * BN), v = i % (KC * BN);
        const float* W = static_cast<const float*>(m == 0 ? p.w0 : p.w1);
        if constexpr (NK) bv[u] = W[((size_t)e * p.N + n0 + v / KC) * p.K + k0 + v % KC];
        else bv[u] = W[((size_t)e * p.K + k0 + v / BN) * p.N + n0 + v % BN];
      }
    };
    load(0);
    for (int k0 = 0; k0 < p.K; k0 += KC) {
#pragma unroll
      for (int u = 0; u < A_PER; ++u) sA[(tid + 256 * u) / KC][(tid + 256 * u) % KC] = av[u];
#pragma unroll
      for (int u = 0; u < B_PER; ++u) {
        const int i = tid + 256 * u;
        const int m = i / (KC * BN), v = i % (KC * BN);
        if constexpr (NK) sB[m][v / KC][v % KC] = bv[u];
        else sB[m][v % BN][v / BN] = bv[u];
      }
      __syncthreads();
      if (k0 + KC < p.K) load(k0 + KC);
#pragma unroll
      for (int kk = 0; kk < KC; kk += 4) {
        const float a0 = sA[li][kk + lk], a1 = sA[16 + li][kk + lk];
#pragma unroll
        for (int m = 0; m < NW; ++m) {
          const float b = sB[m][16 * wave + li][kk + lk];
          acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b, acc[m][0], 0, 0, 0);
          acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b, acc[m][1], 0, 0, 0);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * h + 4 * lk + r;
        if (row >= rows) continue;
        float v;
        if constexpr (GU) v = silu_mul(acc[0][h][r], acc[1][h][r]);
        else v = acc[0][h][r];
        O[(size_t)(row0 + row) * p.N + n0 + 16 * wave + li] = v;
      }
  }
}


template <class C, typename OutT>
hipError_t run_bf16(const GemmParams& p, int wgs_per_cu, hipStream_t s) {
  const size_t lds = C::lds_bytes(p.n_groups);
  // Upper bound of the tile count: every group adds at most one partial m-tile.
  const long long max_tiles = ((long long)(p.rows_cap + C::BM - 1) / C::BM + p.n_groups) * (p.N / C::BN);
  const int fit = (int)(kLdsPerCu / lds);              // workgroups that fit in one CU's LDS (>= 1)
  if (wgs_per_cu > fit) wgs_per_cu = fit;
  long long grid = (long long)device_cu_count() * wgs_per_cu;
  if (grid > max_tiles) grid = max_tiles;
  grid = ((grid + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  if constexpr (C::STAGES == 1 && !C::Q4 && !C::SUM && !C::W8 && !C::KN) {
    if (p.row_index == nullptr && (p.K / C::KC) % 2 == 0) {
      k_gemm_stream<C, OutT><<<dim3((unsigned)grid), dim3(C::NT), lds, s>>>(p);
      return hipGetLastError();
    }
  }
  k_gemm_bf16<C, OutT><<<dim3((unsigned)grid), dim3(C::NT), lds, s>>>(p);
  return hipGetLastError();
}

template <bool GU, bool NK>
hipError_t run_f32(const GemmParams& p, hipStream_t s) {
  const size_t lds = 2 * sizeof(int) * (p.n_groups + 1);
  const long long max_tiles = ((long long)(p.rows_cap + 31) / 32 + p.n_groups) * (p.N / 64);
  long long grid = (long long)device_cu_count() * 4;
  if (grid > max_tiles) grid = max_tiles;
  grid = ((grid + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  k_gemm_f32<GU, NK><<<dim3((unsigned)grid), dim3(256), lds, s>>>(p);
  return hipGetLastError();
}

}  // namespace

// Tile variants, chosen on the host from the shape before anything is launched:
//   0 (decode-shaped, few rows per expert): 32x64 | 32x128 (gate/up | down) tiles, 4 waves (1x4),
//     1 LDS buffer, two chunks in registers, 4 workgroups per CU (dense down: 2 per CU);
//   1 (prefill-shaped): 256x128 | 256x256, 8 waves (4x2), 2 LDS buffers, 1 per CU; dense weights go
//     straight from global memory to LDS (down with up to 64 experts: three weight buffers); int4
//     words go through one register set and are dequantised on the way;
//   2 (prefill-shaped, N not a multiple of variant 1's width): 256x64 | 256x128, 4 waves (4x1),
//     2 LDS buffers, 1 per CU, two chunks in registers.
// Every variant's LDS (two 256-row buffers and a tile table of up to 1024 groups) fits in 160 KB.
namespace {

template <int BM, int BN, int WM, int WN, bool GU>
constexpr bool cfg_ok() {
  constexpr int NT = 64 * WM * WN, NW = GU ? 2 : 1, A_CHUNKS = BM * 8;
  return (WM * WN == 4 || WM * WN == 8) && (NW * 64 * BN) % (32 * NT) == 0 && NW * 64 * BN >= 32 * NT &&
         (A_CHUNKS % NT == 0 || NT % A_CHUNKS == 0) && BM / WM >= 16 && BN / WN >= 16;
}

// Output dtypes of one launch (the ABI's checks leave these combinations):
//   gate/up: bf16 activations; h in bf16 or fp16 (dense weights: bf16 operands; int4: fp16
//            operands, activations converted); int4 needs fp16 h;
//   down:    bf16 h with bf16 weights (bf16 operands) or fp16 h with fp16 or int4 weights (fp16
//            operands); out in fp32 or h's dtype.
template <int BM, int BN, int WM, int WN, int ST, int WGS, int RS, bool Q4, bool F16, typename OutT, bool W8 = false>
hipError_t run_cfg_gu(const GemmParams& p, hipStream_t s) {
  static_assert(cfg_ok<BM, BN, WM, WN, true>(), "gate/up tile");
  using C = Cfg<BM, BN, WM, WN, ST, true, Q4, WGS, RS, F16, F16, false, W8>;
  static_assert(C::STAGES * C::STAGE * 2 + 2 * 4 * 1025 + 16 <= kLdsPerCu, "LDS");
  return run_bf16<C, OutT>(p, WGS, s);
}

template <int BM, int BN, int WM, int WN, int ST, int WGS, int RS, bool Q4, bool F16, typename OutT, bool W8 = false>
hipError_t run_cfg_dn(const GemmParams& p, hipStream_t s) {
  static_assert(cfg_ok<BM, BN, WM, WN, false>(), "down tile");
  using C = Cfg<BM, BN, WM, WN, ST, false, Q4, WGS, RS, F16, false, false, W8>;
  static_assert(C::STAGES * C::STAGE * 2 + 2 * 4 * 1025 + 16 <= kLdsPerCu, "LDS");
  return run_bf16<C, OutT>(p, WGS, s);
}

// gate/up, one tile shape: int4 on fp16 operands (h fp16), or dense bf16 (h bf16 or fp16)
template <int BM, int BN, int WM, int WN, int ST, int WGS, int RS>
hipError_t run_gu_q4(const GemmParams& p, hipStream_t s) {
  return run_cfg_gu<BM, BN, WM, WN, ST, WGS, RS, true, true, _Float16>(p, s);
}
template <int BM, int BN, int WM, int WN, int ST, int WGS, int RS>
hipError_t run_gu(const GemmParams& p, bool q4, bool h16, hipStream_t s) {
  if (q4) return run_gu_q4<BM, BN, WM, WN, ST, WGS, RS>(p, s);
  return h16 ? run_cfg_gu<BM, BN, WM, WN, ST, WGS, RS, false, false, _Float16>(p, s)
             : run_cfg_gu<BM, BN, WM, WN, ST, WGS, RS, false, false, u16>(p, s);
}

// down, one tile shape: operands bf16 (dense bf16) or fp16 (h fp16 with fp16 or int4 weights)
template <int BM, int BN, int WM, int WN, int ST, int WGS, int RS>
hipError_t run_dn(const GemmParams& p, bool q4, bool f16, bool f32out, hipStream_t s) {
  if (q4)
    return f32out ? run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, true, true, float>(p, s)
                  : run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, true, true, _Float16>(p, s);
  if (f16)
    return f32out ? run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, false, true, float>(p, s)
                  : run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, false, true, _Float16>(p, s);
  return f32out ? run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, false, false, float>(p, s)
                : run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, false, false, u16>(p, s);
}

// fp8 weights, one tile shape: gate/up on bf16 operands (h bf16 or fp16); down on the operand type
// of h (bf16 or fp16), out fp32 or h's dtype
template <int BM, int BN, int WM, int WN, int ST, int WGS, int RS>
hipError_t run_gu_w8(const GemmParams& p, bool h16, hipStream_t s) {
  return h16 ? run_cfg_gu<BM, BN, WM, WN, ST, WGS, RS, false, false, _Float16, true>(p, s)
             : run_cfg_gu<BM, BN, WM, WN, ST, WGS, RS, false, false, u16, true>(p, s);
}
template <int BM, int BN, int WM, int WN, int ST, int WGS, int RS>
hipError_t run_dn_w8(const GemmParams& p, bool f16, bool f32out, hipStream_t s) {
  if (f16)
    return f32out ? run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, false, true, float, true>(p, s)
                  : run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, false, true, _Float16, true>(p, s);
  return f32out ? run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, false, false, float, true>(p, s)
                : run_cfg_dn<BM, BN, WM, WN, ST, WGS, RS, false, false, u16, true>(p, s);
}

// dense prefill-shaped down projection with direct global -> LDS loads
template <bool F16, typename OutT>
hipError_t run_dma_dn(const GemmParams& p, hipStream_t s) {
  using D = DCfg<256, 256, 4, 2, false, F16>;
  if (p.n_groups <= 64) return run_dma3<D, OutT>(p, s);   // tile table in registers: three weight buffers
  return run_dma<D, OutT>(p, s);
}

}  // namespace

hipError_t launch_grouped_gemm(const moe_gemm_args& a, hipStream_t s) {
  GemmParams p;
  p.a = a.a; p.row_index = a.row_index; p.group_offsets = a.group_offsets;
  p.w0 = a.w0; p.w1 = a.w1; p.s0 = a.s0; p.s1 = a.s1; p.out = a.out; p.bias = nullptr;
  p.K = a.K; p.N = a.N; p.n_groups = a.n_groups; p.rows_cap = a.rows_cap; p.a_rows = a.a_rows;
  p.row_div = a.row_div; p.group_size = a.group_size > 0 ? a.group_size : a.K;
  const bool gu = a.op == MOE_OP_GATE_UP_SWIGLU;
  if (a.act_dtype == MOE_DT_F32) {
    const bool nk = a.wfmt == MOE_W_DENSE_NK;
    return gu ? (nk ? run_f32<true, true>(p, s) : run_f32<true, false>(p, s))
              : (nk ? run_f32<false, true>(p, s) : run_f32<false, false>(p, s));
  }
  const bool q4 = a.wfmt == MOE_W_INT4_SYM_GROUP;
  const bool f16 = q4 || a.act_dtype == MOE_DT_F16;    // fp16 operands
  const bool f32out = a.out_dtype == MOE_DT_F32;
  const bool h16 = a.out_dtype == MOE_DT_F16;
  // The ABI guarantees N % 64 == 0 (gate/up) and N % 128 == 0 (down): variants 0 and 2 always fit.
  const bool small_m = a.m_hint > 0 && a.m_hint <= 48;   // decode-shaped: weight streaming
  const bool k4 = p.K % 256 == 0;                       // four 64-k chunks per register round
  if (a.wfmt == MOE_W_DENSE) {
    // bf16 weights in the stated [e][K][N] layout: register-staged tiles with transposed operand
    // reads (the prepared [e][N][K] copy takes the faster paths below)
    if (gu) {
      if (small_m) return h16 ? run_bf16<Cfg<32, 64, 1, 4, 1, true, false, 4, 2, false, false, false, false, true>, _Float16>(p, 4, s)
                              : run_bf16<Cfg<32, 64, 1, 4, 1, true, false, 4, 2, false, false, false, false, true>, u16>(p, 4, s);
      return h16 ? run_bf16<Cfg<256, 64, 4, 1, 2, true, false, 1, 2, false, false, false, false, true>, _Float16>(p, 1, s)
                 : run_bf16<Cfg<256, 64, 4, 1, 2, true, false, 1, 2, false, false, false, false, true>, u16>(p, 1, s);
    }
    if (small_m) return f32out ? run_bf16<Cfg<32, 128, 1, 4, 1, false, false, 2, 2, false, false, false, false, true>, float>(p, 2, s)
                               : run_bf16<Cfg<32, 128, 1, 4, 1, false, false, 2, 2, false, false, false, false, true>, u16>(p, 2, s);
    return f32out ? run_bf16<Cfg<256, 128, 4, 1, 2, false, false, 1, 2, false, false, false, false, true>, float>(p, 1, s)
                  : run_bf16<Cfg<256, 128, 4, 1, 2, false, false, 1, 2, false, false, false, false, true>, u16>(p, 1, s);
  }
  if (a.wfmt == MOE_W_FP8_E4M3) {
    if (gu) {
      if (small_m) return k4 ? run_gu_w8<32, 64, 1, 4, 1, 4, 4>(p, h16, s) : run_gu_w8<32, 64, 1, 4, 1, 4, 2>(p, h16, s);
      if (p.N % 128 == 0) return run_gu_w8<192, 128, 4, 2, 2, 1, 1>(p, h16, s);
      return run_gu_w8<256, 64, 4, 1, 2, 1, 2>(p, h16, s);
    }
    if (small_m)
      return k4 ? run_dn_w8<32, 128, 1, 4, 1, 4, 4>(p, f16, f32out, s) : run_dn_w8<32, 128, 1, 4, 1, 4, 2>(p, f16, f32out, s);
    // 8-wave 192 x 256 tiles (256 rows need more than two waves' registers per SIMD)
    if (p.N % 256 == 0) return run_dn_w8<192, 256, 4, 2, 2, 1, 1>(p, f16, f32out, s);
    return run_dn_w8<256, 128, 4, 1, 2, 1, 2>(p, f16, f32out, s);
  }
  if (gu) {
    if (small_m) {
      if (q4 && k4) return run_gu_q4<32, 64, 1, 4, 1, 4, 4>(p, s);
      return run_gu<32, 64, 1, 4, 1, 4, 2>(p, q4, h16, s);
    }
    if (p.N % 128 == 0) {
      // int4: 192-row tiles (256 rows need more than the 256 registers of two waves per SIMD)
      if (q4) return run_gu_q4<192, 128, 4, 2, 2, 1, 1>(p, s);
      return h16 ? run_dma<DCfg<256, 128, 4, 2, true>, _Float16>(p, s) : run_dma<DCfg<256, 128, 4, 2, true>, u16>(p, s);
    }
    return run_gu<256, 64, 4, 1, 2, 1, 2>(p, q4, h16, s);
  }
  if (small_m) {
    // dense: two workgroups per CU (half as many weight streams, each workgroup streams several
    // tiles back to back): 2 % faster than four on the decode-shaped down projection
    if (q4) {
      // four register sets with fp16 output; otherwise two, at three workgroups per CU (the fp32
      // epilogue and the activation reordering of int4 tiles need more than a quarter of the
      // registers)
      if (k4 && !f32out) return run_cfg_dn<32, 128, 1, 4, 1, 4, 4, true, true, _Float16>(p, s);
      return run_dn<32, 128, 1, 4, 1, 3, 2>(p, q4, f16, f32out, s);
    }
    return run_dn<32, 128, 1, 4, 1, 2, 2>(p, q4, f16, f32out, s);
  }
  if (p.N % 256 != 0) return run_dn<256, 128, 4, 1, 2, 1, 2>(p, q4, f16, f32out, s);
  // int4: 192-row tiles (the 256-row tile sits at the 256 registers of two waves per SIMD)
  if (q4) return f32out ? run_cfg_dn<192, 256, 4, 2, 2, 1, 1, true, true, float>(p, s)
                        : run_cfg_dn<192, 256, 4, 2, 2, 1, 1, true, true, _Float16>(p, s);
  if (f16) return f32out ? run_dma_dn<true, float>(p, s) : run_dma_dn<true, _Float16>(p, s);
  return f32out ? run_dma_dn<false, float>(p, s) : run_dma_dn<false, u16>(p, s);
}

// ---------------------------------------------------------------------------------------------
// Router projection: logits = x W_r (+ bias), W_r held as two bf16 planes W_hi + W_lo
// ---------------------------------------------------------------------------------------------
namespace {

// fp32 path (fp32 activations, or E not a multiple of 64): one thread per (token, expert), the
// K sum in order with fma; W_hi + W_lo is exact in fp32.
__global__ __launch_bounds__(256) void k_router_f32(const void* __restrict__ x, int x_bf16, const u16* __restrict__ w,
                                                    const float* __restrict__ bias, int T, int H, int E,
                                                    float* __restrict__ logits) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const u16* hi = w + (size_t)e * H;
  const u16* lo = w + ((size_t)E + e) * H;
  float acc = 0.0f;
  for (int h = 0; h < H; ++h) {
    const float xv = x_bf16 ? bf16_to_f32(static_cast<const u16*>(x)[(size_t)t * H + h])
                            : static_cast<const float*>(x)[(size_t)t * H + h];
    acc = fmaf(xv, bf16_to_f32(hi[h]) + bf16_to_f32(lo[h]), acc);
  }
  if (bias) acc = acc + bias[e];
  logits[i] = acc;
}

}  // namespace

hipError_t launch_router_logits(const void* x, int x_dtype, const void* w_split, const float* bias, int T, int H,
                                int E, float* logits, hipStream_t s) {
  if (x_dtype != MOE_DT_BF16 || E % 64 != 0 || H % 64 != 0) {
    const long long n = (long long)T * E;
    k_router_f32<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(x, x_dtype == MOE_DT_BF16, static_cast<const u16*>(w_split),
                                                                   bias, T, H, E, logits);
    return hipGetLastError();
  }
  GemmParams p;
  p.a = x; p.row_index = nullptr; p.group_offsets = nullptr;    // one group of T identity rows
  p.w0 = w_split; p.w1 = static_cast<const u16*>(w_split) + (size_t)E * H;
  p.s0 = p.s1 = nullptr; p.out = logits; p.bias = bias;
  p.K = H; p.N = E; p.n_groups = 1; p.rows_cap = T; p.a_rows = T; p.row_div = 1; p.group_size = H;
  // 256-row tiles (64 experts wide) when they give every compute unit about one tile, else
  // 16-row tiles, four workgroups per compute unit, four chunks in registers: with few tiles each
  // workgroup's chain of K chunks is the time, and deeper loads shorten it (decode shape 32.6 ->
  // 27.1 us against 32-row tiles with two chunks)
  const long long big_tiles = (long long)((T + 255) / 256) * (E / 64);
  if (2 * big_tiles >= device_cu_count())
    return run_bf16<Cfg<256, 64, 4, 1, 2, true, false, 1, 2, false, false, true>, float>(p, 1, s);
  if (H % 256 == 0)
    return run_bf16<Cfg<16, 64, 1, 4, 1, true, false, 4, 4, false, false, true>, float>(p, 4, s);
  return run_bf16<Cfg<32, 64, 1, 4, 1, true, false, 4, 2, false, false, true>, float>(p, 4, s);
}

}  // namespace moe
