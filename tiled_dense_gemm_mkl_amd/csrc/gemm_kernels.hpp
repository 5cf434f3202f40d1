// gemm_kernels.hpp -- device code of the gfx950 (CDNA4) tiled dense GEMM.
//
//   C[l][m][n] = epilogue( sum_k A[l][m][k] * B[l][n][k] )
//
// A is [L][M][K], B is [L][N][K] (K contiguous), C is [L][M][N]; the modes are
// those of the persistent dense GEMM on "深入解析 CUTLASS CuTe DSL 的 JIT 函数参数生成机制"
// (section 2.3).  The hot path of one workgroup:
//
//   1. tile mapping: workgroup id -> (batch l, split s, BM x BN output tile),
//      remapped so that consecutive tiles run on the same XCD (shared L2);
//      the output-tile-to-workgroup lift is the tileify / blockify_launch step
//      of "一个可定制的编译器，用于为AI模型生成高效的融合GPU内核" (its Tile-IR pass list).
//   2. K chunking: K is cut into chunks of 128 bytes per row (BK = 64 for
//      16-bit types, 32 for fp32); chunks are the "K-outer" loop and the
//      64-byte MFMA k-steps inside a chunk the "K-inner" loop (chunk_matmul_k
//      in the same list).  With split-K, ranges of chunks become a grid
//      dimension (split_matmul_k).
//   3. LDS staging: every chunk of the A and B tiles is copied to LDS by
//      direct global->LDS buffer loads (16 bytes a lane), in a row-major
//      [rows][128 B] layout whose 16-byte columns are XOR-swizzled by the row
//      index, so that the MFMA operand reads are free of bank conflicts
//      (stage_inputs / split_inner_for_swizzle / pad_smem in the list above).
//   4. A ring of prefetch_stages + 1 LDS slots: the prologue issues chunks
//      0..P-1; iteration i waits for chunk i, then issues chunk i+P into the
//      slot that chunk i-1 used, then computes on chunk i.  This is the
//      manual software pipeline of section 3 of "CUTLASS CuTe DSL 控制流编程指南"
//      (prefetch loop, then a main loop that prefetches i + prefetch_stages
//      while it uses slot i mod stages).  P = 0 is load-then-use.
//   5. MFMA mainloop with fp32 accumulators (v_mfma_f32_16x16x32_{bf16,f16},
//      v_mfma_f32_16x16x4_f32); the operands are swapped (B tile as the MFMA's
//      first operand) so that each lane ends up owning 4 consecutive n.
//   6. Epilogue fused at compile time (identity / ReLU / SiLU, sections 2.3
//      and 7 of the two CuTe DSL pages) on the fp32 sum, then one rounding to
//      the output type; or, for split-K, an fp32 partial tile that the reduce
//      kernel sums in ascending split order before the same epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gmk {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

enum Mode { MODE_IDENTITY = 0, MODE_RELU = 1, MODE_SILU = 2, MODE_PARTIAL = 3 };

// A voffset at or above every buffer's num_records: the load returns zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// n / d for 32-bit unsigned n and 1 <= d < 2^31 by one multiply-high and two
// shifts: division by an invariant integer (Granlund and Montgomery,
// "Division by Invariant Integers using Multiplication", PLDI 1994, section
// 4).  With l = ceil(log2 d) and mul = floor(2^32 (2^l - d) / d) + 1:
//   t = (mul * n) >> 32,   n / d = (t + ((n - t) >> sh1)) >> sh2,
// sh1 = min(l, 1), sh2 = max(l - 1, 0) (d = 1 gives mul = 1, t = 0).  On the
// GPU every step of it is a scalar instruction, where a plain division goes
// through the vector unit's float reciprocal and back.
struct FastDiv {
    uint32_t mul, sh1, sh2;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    FastDiv f;
    f.mul = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    f.sh1 = l < 1 ? l : 1;
    f.sh2 = l > 1 ? l - 1 : 0;
    return f;
}

__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f)
{
    const uint32_t t = (uint32_t)(((uint64_t)f.mul * n) >> 32);
    return (t + ((n - t) >> f.sh1)) >> f.sh2;
}

// Workgroup -> (batch, split, tile row, tile column) of the data-parallel
// grid, every division precomputed by the host (make_tile_map).
//   - Hardware dispatches consecutive workgroup ids round-robin over the 8
//     XCDs.  The full rounds are renumbered so that each XCD holds a
//     contiguous range of ids (the ragged last round keeps its ids); the id
//     is then split [batch][split][tile].
//   - Blocked grids (one batch, no split, an even number of tile rows, tile
//     columns a multiple of 4, at least 512 tiles): XCD x = id % 8 walks
//     block (x / 4, x % 4) of a 2 x 4 cut of the tile grid, so that it reads
//     only that block's rows of A and columns of B instead of every column
//     of B (measured on fp16 8192^3: 913 -> 892 us).
//   - Tiles are rastered, over the grid or the block, in groups of `group`
//     tile rows, column-major inside a group (tiles sharing B columns run
//     together and share the L2).
struct TileMap {
    int32_t per;                  // full rounds of the 8 XCDs: grid / 8
    int32_t tiles, split;         // tiles of one batch; K splits
    FastDiv d_tiles, d_split;
    int32_t blocked;
    int32_t rows, cols;           // the rastered area: the grid, or one block
    int32_t group, last_first;    // tile rows per group; first row of the last group
    FastDiv d_width, d_group, d_last;   // by group * cols, group, rows of the last group
};

// (row, column) of tile `tile` of the rastered area.
__host__ __device__ __forceinline__ void raster_map(const TileMap &m, uint32_t tile, int &r, int &c)
{
    const uint32_t gi = fdiv(tile, m.d_width);
    const int first = (int)gi * m.group;
    const bool last = first >= m.last_first;
    const int gsize = last ? m.rows - first : m.group;
    const uint32_t u = tile - gi * (uint32_t)(m.group * m.cols);
    const uint32_t q = fdiv(u, last ? m.d_last : m.d_group);
    r = first + (int)(u - q * (uint32_t)gsize);
    c = (int)q;
}

// Branch-free, so that the compiler loads every field in one round of kernel
// argument loads.  In a blocked grid the id within the XCD's block,
// b / 8 < tiles, gives batch and split 0 by the same divisions.
__host__ __device__ __forceinline__ void map_workgroup(const TileMap &m, uint32_t b, int &l, int &s, int &tm,
                                                       int &tn)
{
    const uint32_t per = (uint32_t)m.per;
    const uint32_t remapped = b < 8u * per ? (b & 7) * per + (b >> 3) : b;
    const uint32_t t = m.blocked ? (b >> 3) : remapped;
    const uint32_t q = fdiv(t, m.d_tiles);
    const uint32_t lq = fdiv(q, m.d_split);
    l = (int)lq;
    s = (int)(q - lq * (uint32_t)m.split);
    raster_map(m, t - q * (uint32_t)m.tiles, tm, tn);
    tm += m.blocked ? (int)((b & 7) >> 2) * m.rows : 0;
    tn += m.blocked ? (int)(b & 3) * m.cols : 0;
}

// The map of a grid of `grid` workgroups over L batches, `split` K splits and
// tiles_m x tiles_n tiles, rastered in groups of group_m tile rows.
inline TileMap make_tile_map(int tiles_m, int tiles_n, int L, int split, int group_m, int grid)
{
    TileMap m;
    m.per = grid / 8;
    m.tiles = tiles_m * tiles_n;
    m.split = split;
    m.d_tiles = make_fastdiv((uint32_t)m.tiles);
    m.d_split = make_fastdiv((uint32_t)split);
    m.blocked = (L == 1 && split == 1 && tiles_m % 2 == 0 && tiles_n % 4 == 0 && m.tiles >= 512) ? 1 : 0;
    m.rows = m.blocked ? tiles_m / 2 : tiles_m;
    m.cols = m.blocked ? tiles_n / 4 : tiles_n;
    m.group = group_m < 1 ? 1 : (group_m > m.rows ? m.rows : group_m);
    m.last_first = (m.rows - 1) / m.group * m.group;
    m.d_width = make_fastdiv((uint32_t)(m.group * m.cols));
    m.d_group = make_fastdiv((uint32_t)m.group);
    m.d_last = make_fastdiv((uint32_t)(m.rows - m.last_first));
    return m;
}

struct TileParams {
    const void *A;
    const void *B;
    void *C;          // output (modes 0..2) or fp32 workspace [S][L][M][N] (partial)
    int64_t M, N, K, L;
    int32_t tiles_m, tiles_n;
    int32_t group_m;          // tile rows per raster group (L2 reuse)
    int32_t split;            // S
    int32_t chunks_per_split; // K chunks per split (the last split may be short)
    int32_t total_chunks;     // ceil(K * elem / row bytes of a chunk)
    TileMap map;              // the data-parallel grid's workgroup -> tile map
};

// ------------------------------------------------------------------ epilogue

template <int MODE>
__device__ __forceinline__ float apply_epilogue(float x)
{
    if constexpr (MODE == MODE_RELU) {
        return x > 0.0f ? x : 0.0f;          // where(x > 0, x, 0): -0 and NaN give +0
    } else if constexpr (MODE == MODE_SILU) {
        return x / (1.0f + expf(-x));        // x * sigmoid(x)
    } else {
        return x;
    }
}

// ------------------------------------------------------------------ element types

template <class T> struct Elem;

template <> struct Elem<float> {
    static constexpr int bytes = 4;
    __device__ static __forceinline__ f32x4 mfma_step(i32x4 a, i32x4 b, f32x4 acc)
    {
        // one 16-byte read holds 4 consecutive k of a row: four 16x16x4 MFMAs,
        // MFMA j taking component j on both operands (same k on both sides)
        f32x4v av = __builtin_bit_cast(f32x4v, a);
        f32x4v bv = __builtin_bit_cast(f32x4v, b);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bv[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bv[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bv[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], bv[3], acc, 0, 0, 0);
        return acc;
    }
    __device__ static __forceinline__ float from_f32(float x) { return x; }
    __device__ static __forceinline__ float to_f32(float x) { return x; }
    __device__ static __forceinline__ void store4(float *p, float a, float b, float c, float d)
    {
        f32x4v v = {a, b, c, d};
        *reinterpret_cast<f32x4v *>(p) = v;
    }
};

template <> struct Elem<__bf16> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ f32x4 mfma_step(i32x4 a, i32x4 b, f32x4 acc)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ __bf16 from_f32(float x) { return (__bf16)x; }  // RNE
    __device__ static __forceinline__ float to_f32(__bf16 x) { return (float)x; }
    __device__ static __forceinline__ void store4(__bf16 *p, float a, float b, float c, float d)
    {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
        *reinterpret_cast<bf16x4 *>(p) = v;
    }
};

template <> struct Elem<_Float16> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ f32x4 mfma_step(i32x4 a, i32x4 b, f32x4 acc)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ _Float16 from_f32(float x) { return (_Float16)x; }  // RNE
    __device__ static __forceinline__ float to_f32(_Float16 x) { return (float)x; }
    __device__ static __forceinline__ void store4(_Float16 *p, float a, float b, float c, float d)
    {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        f16x4 v = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
        *reinterpret_cast<f16x4 *>(p) = v;
    }
};

// ------------------------------------------------------------------ low-level helpers

// Buffer resource for raw (unswizzled) addressing; out-of-range reads return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_records)
{
    uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
    r[3] = 0x00020000;                                               // gfx9 data format word
    return r;
}

// Direct global->LDS loads of 16 bytes per lane.  Lane t of a load writes LDS
// bytes [M0 + OFF + 16 t, M0 + OFF + 16 t + 16) with the 16 global bytes at
// rsrc.base + voffset + soffset + OFF; the instruction offset OFF (0, 1024,
// 2048 or 3072 here) moves both addresses.  Writing M0 costs far more than the
// load itself, so one M0 value serves four consecutive 1 KB blocks.  The loads
// are inline asm so that the compiler adds no conservative waits for them;
// the ring waits on vmcnt explicitly.  A write of M0 needs one wait state
// before an LDS-DMA instruction reads it, hence the s_nop.
// Every one of these statements lists M0 as clobbered: the compiler then
// never assigns one of their operands to M0 and never keeps a value of its
// own in M0 across them.  The M0 that dma16_same_m0 reads is the one the last
// dma16_set_m0 wrote; the compiled kernels contain no other write of M0
// between the two (the ISA has no M0 write that is not one of ours).
__device__ __forceinline__ void dma16_set_m0(i32x4 rsrc, uint32_t m0, uint32_t voffset, uint32_t soffset)
{
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voffset), "s"(rsrc), "s"(soffset)
                 : "memory", "m0");
}

// Load block j (1..3) of the four sharing the current M0.
__device__ __forceinline__ void dma16_same_m0(i32x4 rsrc, int j, uint32_t voffset, uint32_t soffset)
{
    switch (j) {
    case 1:
        asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:1024 lds" : : "v"(voffset), "s"(rsrc), "s"(soffset)
                     : "memory", "m0");
        break;
    case 2:
        asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:2048 lds" : : "v"(voffset), "s"(rsrc), "s"(soffset)
                     : "memory", "m0");
        break;
    default:
        asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:3072 lds" : : "v"(voffset), "s"(rsrc), "s"(soffset)
                     : "memory", "m0");
        break;
    }
}

// The global side of a block j load gets OFF = (j % 4) * 1024 added; the
// resource base sits kRsrcBias bytes before the tile and every voffset carries
// kRsrcBias - OFF, so the byte read is exactly the intended one and voffset
// never goes negative.
constexpr uint32_t kRsrcBias = 4096;

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier that first drains this wave's LDS reads.  No vmcnt wait:
// prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// Plain workgroup barrier (the waves' own waits precede it).
__device__ __forceinline__ void block_barrier()
{
    asm volatile("s_barrier" : : : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// Workgroup id -> logical tile id.  Hardware dispatches consecutive workgroup
// ids round-robin over the 8 XCDs; this gives each XCD a contiguous range of
// logical ids so that tiles sharing A rows or B columns share one L2.
__device__ __forceinline__ int xcd_remap(int wg, int grid)
{
    constexpr int kXcd = 8;
    int per = grid / kXcd;            // full rounds
    int full = per * kXcd;
    if (wg >= full) return wg;        // the ragged last round keeps its ids
    return (wg % kXcd) * per + wg / kXcd;
}

// Tile id (within one batch) -> (tm, tn): tiles rastered in groups of group_m
// tile rows, column-major inside a group.
__device__ __forceinline__ void raster(int tile, int tiles_m, int tiles_n, int group_m, int &tm, int &tn)
{
    const int width = group_m * tiles_n;
    const int first_m = (tile / width) * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    tm = first_m + (tile % width) % gsize;
    tn = (tile % width) / gsize;
}

// ------------------------------------------------------------------ the tiled kernel

// LDS row layout of one chunk: RB bytes per row (64 or 128), split in 16-byte
// columns.  Column c of row r is stored at physical column c ^ swizzle(r),
// chosen for the read pattern of the MFMA shape MF (a 16-byte read per lane):
//   RB = 128, MF = 32 (32 rows x 2 columns per read):
//       swizzle(r) = (r & 7) ^ ((r >> 3) & 1)
//   RB = 128, MF = 16 (16 rows x 4 columns per read): swizzle(r) = r & 7
//   RB =  64, MF = 32 (32 rows x 2 columns per read): swizzle(r) = (r >> 2) & 3
// Measured with a read-throughput probe (16 waves per CU): each form reads
// at the rate of a linear 1 KB read (about 5 clocks per instruction per CU);
// the MF = 32 form applied to the MF = 16 pattern takes 8 (a 2-way bank
// conflict on every read), and no swizzle takes 16.
template <int RB, int MF>
__device__ __forceinline__ int row_swizzle(int r)
{
    if constexpr (RB == 128 && MF == 16)
        return r & 7;
    else if constexpr (RB == 128)
        return (r & 7) ^ ((r >> 3) & 1);
    else
        return (r >> 2) & 3;
}

// Cache policy of the stream-K partial tiles: SC0 | SC1 (system scope), so the
// stores write through to memory and the loads do not hit a stale line in
// another XCD's L2; no L2-wide write-back or invalidate is needed.
constexpr int kCoherent = 1 | 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const float *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, 0x7fffffff, 0x00020000);
}

template <class T, int MF> struct Mfma;

template <class T> struct Mfma<T, 16> {
    typedef f32x4 acc_t;
    static constexpr int regs = 4;
    __device__ static __forceinline__ acc_t step(i32x4 a, i32x4 b, acc_t c) { return Elem<T>::mfma_step(a, b, c); }
};

template <class T> struct Mfma<T, 32> {
    typedef float acc_t __attribute__((ext_vector_type(16)));
    static constexpr int regs = 16;
    __device__ static __forceinline__ acc_t step(i32x4 a, i32x4 b, acc_t c)
    {
        if constexpr (sizeof(T) == 4) {
            // 16 bytes = 4 consecutive k of a row: four 32x32x2 MFMAs, MFMA j taking
            // component j on both operands
            f32x4v av = __builtin_bit_cast(f32x4v, a);
            f32x4v bv = __builtin_bit_cast(f32x4v, b);
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[0], bv[0], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[1], bv[1], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[2], bv[2], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[3], bv[3], c, 0, 0, 0);
            return c;
        } else if constexpr (__is_same(T, __bf16)) {
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                           c, 0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                          c, 0, 0, 0);
        }
    }
};

// The work of one workgroup on one BM x BN tile of C: buffer descriptors and
// per-lane load offsets for the tile, the prefetch ring over a range of K
// chunks into fp32 accumulators, and the stores of the result.
//   RB      bytes of K per row in one chunk (the K-outer step)
//   MF      MFMA block edge: 32 (v_mfma_f32_32x32x16 / 32x32x2f32) or 16
//   P       prefetch_stages: chunks in flight ahead of the one consumed
//   WK      wave groups along K: group kg computes the whole wave tile over
//           its share of every chunk's k-steps (k-steps kg * KSW .. + KSW - 1),
//           so each group reads each operand fragment once; the groups' sums
//           are added in ascending kg before the epilogue.  A chunk's LDS
//           reads per MFMA fall by WK at the cost of one cross-wave reduction.
//   NP      producer waves (0: every wave loads and computes).  With NP > 0
//           the NP extra waves issue all global->LDS loads and the MFMA waves
//           only read LDS and compute: a direct-to-LDS load stalls the wave
//           that issues it for many cycles when the address unit is busy,
//           which costs a computing wave its MFMA slots but costs a producer
//           nothing.  Needs P >= 2.
//   ILV     interleaved row blocks: fragment row i of wave row wm covers tile
//           rows (i * WAVES_M + wm) * MF .. + MF - 1 (else wm * WTM + i * MF ..),
//           so that the live rows of a partly filled tile are shared out
//           evenly over the wave rows, and the MFMAs of whole MF-row blocks
//           past the last row can be skipped (run_live).
template <class T, int BM, int BN, int RB, int WAVES_M, int WAVES_N, int MF, int P, int WK = 1, int NP = 0,
          bool ILV = false>
struct TileCore {
    typedef Mfma<T, MF> MM;
    typedef typename MM::acc_t acc_t;
    static constexpr int NWT = WAVES_M * WAVES_N;        // waves of one k-group
    static constexpr int NWM = NWT * WK;                 // MFMA waves
    static constexpr int NW = NWM + NP;
    static constexpr int NL = NP > 0 ? NP : NW;          // waves that issue the loads
    static constexpr int THREADS = NW * 64;
    static constexpr int ES = Elem<T>::bytes;
    static constexpr int NCH = RB / 16;                  // 16-byte columns per row
    static constexpr int ROWS_PER_LOAD = 1024 / RB;      // rows covered by one 64-lane 16-byte load
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int FM = WTM / MF;
    static constexpr int FN = WTN / MF;
    static constexpr int STEP_COLS = 64 / MF;            // 16-byte columns one MFMA k-step reads per row
    static constexpr int KSTEPS = NCH / STEP_COLS;       // MFMA k-steps of a chunk
    static constexpr int KSW = KSTEPS / WK;              // ... per wave
    static constexpr int SLOTS = P + 1;
    static constexpr int SLOT_BYTES = (BM + BN) * RB;
    static constexpr int LDS_BYTES = SLOTS * SLOT_BYTES;
    static constexpr int A_GROUPS = BM / ROWS_PER_LOAD;
    static constexpr int B_GROUPS = BN / ROWS_PER_LOAD;
    static constexpr int A_LOADS = A_GROUPS / NL;
    static constexpr int B_LOADS = B_GROUPS / NL;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static constexpr int FRAG_ROWS = ILV ? WAVES_M * MF : MF;   // tile rows between fragment rows i, i + 1
    static constexpr int NMF = FM * FN;                  // MFMAs per k-step
    static constexpr int NRD = FM + FN;                  // fragment reads per k-step
    static constexpr int NREG = FM * FN * MM::regs;      // accumulator floats per lane
    // Fragment reads run RA k-steps ahead of their MFMAs, in a ring of NB = RA + 1
    // register buffers: one k-step of MFMAs covers the LDS latency when it holds
    // at least 8 MFMAs; smaller wave tiles read KSW - 1 steps ahead.
    static constexpr int RA = (NMF >= 8 || KSW < 4) ? 1 : KSW - 1;
    static constexpr int NB = RA + 1;
    static_assert(KSW % NB == 0, "fragment ring must divide a wave's k-steps of a chunk");
    // Every wave loads (NP == 0), P >= 2: one wait and one barrier per chunk,
    // at the chunk boundary.  At
    // the end of chunk i every wave has issued all MFMAs of chunk i (so its
    // reads of slot i are complete) and chunk i + 2 must be visible (its first
    // RA k-steps are read during chunk i + 1); the loads of chunk i + 1 + P,
    // spread over all k-steps of chunk i + 1, then refill slot i.  In flight
    // at the wait: the loads of chunks i + 3 .. i + P.
    // NP == 0, P == 1: chunk i + 1 is loaded during chunk i itself, so it is waited for
    // at k-step WIN = KSW - RA of chunk i, just before its first reads; the
    // loads all go out in k-step 0, between its MFMAs, to give them the most
    // time before the wait (measured against spreading them over the k-steps
    // before it: fp16 8192^3 870 -> 857 us, bf16 4096^3 106.1 -> 104.0 us),
    // and the barrier there also drains this wave's reads of chunk i (slot
    // i - 1 ... is refilled from the next chunk on).
    static constexpr int WIN = KSW - RA;
    // Producer ring (NP > 0): where the MFMA waves meet the producers.
    //   WIN_MEET (P <= 3): once per chunk at k-step WIN, where the MFMA waves'
    //   reads move from chunk i to chunk i + 1; that barrier drains their LDS
    //   reads, so slot i is free and chunk i + 1 must have landed.  Right
    //   after it the producers issue chunk i + SLOTS into slot i: every chunk
    //   has P chunk times to arrive.
    //   Otherwise: once per chunk at its end, where every MFMA of chunk i is
    //   issued (its reads of slot i have completed, no drain); the producers
    //   then issue chunk i + P into the slot of chunk i - 1 and wait for chunk
    //   i + 2 (whose first RA k-steps are read during chunk i + 1): P - 1
    //   chunk times.
    // Measured on 512 x 5632 x 2048 bf16 (interleaved, one box): depth 2 on
    // 128 x 256 tiles 30.5 us at the chunk end against 21.4 us at WIN; depth 3
    // on 128 x 192 20.2 against 20.0; depth 4 on 128 x 128 16.7 against
    // 17.3 (and 1024 x 5632 x 8192: 99 against 102), where the drain at WIN
    // costs more than the longer time to arrive gains.
    static constexpr bool WIN_MEET = P <= 3;
    static constexpr int SPREAD = P >= 2 ? KSW : 1;
    static constexpr int LPK = (LOADS + SPREAD - 1) / SPREAD;      // loads per k-step
    static constexpr int WAIT_CNT = P >= 2 ? LOADS * (P - 2) : 0;
    static_assert(RB == 64 || RB == 128, "row bytes");
    static_assert(MF == 16 || MF == 32, "MFMA shape");
    static_assert(BM % (MF * WAVES_M) == 0 && BN % (MF * WAVES_N) == 0, "wave tile");
    static_assert(A_GROUPS % NL == 0 && B_GROUPS % NL == 0, "load split");
    static_assert(NP == 0 || P >= 2, "producer waves need a ring of at least 3 slots");
    static_assert(KSTEPS % WK == 0 && KSW >= 2 && KSW % 2 == 0,
                  "k-steps per wave and chunk: even, for the register double buffer");
    static_assert(WK == 1 || NWT * NREG * 256 <= LDS_BYTES, "LDS for the cross-group reduction");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 workgroup");
    static_assert(LOADS * (P > 0 ? P : 1) < 64, "vmcnt range");
    static_assert(NP == 0 || LOADS * (P + 1) < 64, "vmcnt range of the producer ring (up to P + 1 chunks in flight)");

    char *smem;
    uint32_t smem_base;
    int lane, wave, wm, wn, kg, li, lrow, lcol, sw;
    bool mma;   // an MFMA wave (else a producer)
    uint32_t rd_a, rd_b;
    int64_t m0, n0, k_bytes;
    int l;
    i32x4 rsrc_a, rsrc_b;
    uint32_t voff_a[A_LOADS], voff_b[B_LOADS];
    int col_a[A_LOADS], col_b[B_LOADS];
    acc_t acc[FM][FN];
    i32x4 fa[NB][FM], fb[NB][FN];

    __device__ __forceinline__ void init(char *lds)
    {
        smem = lds;
        smem_base = lds_addr(lds);
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        mma = wave < NWM;
        li = NP == 0 ? wave : (mma ? 0 : wave - NWM);   // loader index (producers: 0 .. NP - 1)
        kg = wave / NWT;
        wm = (wave % NWT) % WAVES_M;
        wn = (wave % NWT) / WAVES_M;
        // operand reads: lane reads row (lane % MF) of each fragment at logical
        // column ks * STEP_COLS + lane / MF
        lrow = lane % MF;
        lcol = lane / MF;
        sw = row_swizzle<RB, MF>(lrow);
        rd_a = (uint32_t)((row_block(0) + lrow) * RB);
        rd_b = (uint32_t)(BM * RB + (wn * WTN + lrow) * RB);
    }

    // First tile row of fragment row i of this wave.
    __device__ __forceinline__ int row_block(int i) const
    {
        return ILV ? (i * WAVES_M + wm) * MF : wm * WTM + i * MF;
    }

    // Buffer descriptors and per-lane offsets for tile (l, tm, tn).
    __device__ __forceinline__ void setup(const TileParams &p, int l_, int tm, int tn)
    {
        l = l_;
        m0 = (int64_t)tm * BM;
        n0 = (int64_t)tn * BN;
        const int64_t K = p.K;
        k_bytes = K * ES;
        const T *Ab = reinterpret_cast<const T *>(p.A) + ((int64_t)l * p.M + m0) * K;
        const T *Bb = reinterpret_cast<const T *>(p.B) + ((int64_t)l * p.N + n0) * K;
        const int64_t rows_a = p.M - m0;
        const int64_t rows_b = p.N - n0;
        // the descriptors start kRsrcBias bytes early (see dma16_same_m0);
        // nothing is ever read there, and the range check still ends at the
        // tile's last row
        const int64_t lim_a = rows_a * k_bytes + kRsrcBias, lim_b = rows_b * k_bytes + kRsrcBias;
        rsrc_a = make_rsrc(reinterpret_cast<const char *>(Ab) - kRsrcBias,
                           (uint32_t)(lim_a < (int64_t)kOutOfRange ? lim_a : kOutOfRange));
        rsrc_b = make_rsrc(reinterpret_cast<const char *>(Bb) - kRsrcBias,
                           (uint32_t)(lim_b < (int64_t)kOutOfRange ? lim_b : kOutOfRange));
        // Wave w loads the row groups [w * A_LOADS, (w + 1) * A_LOADS) of A
        // (and likewise of B), so that its blocks are contiguous in LDS;
        // lane -> (row lane / NCH of the group, physical column lane % NCH,
        // holding logical column that ^ swizzle(row)).
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j) {
            const int g = li * A_LOADS + j;
            const int r = g * ROWS_PER_LOAD + lane / NCH;
            const int c = (lane % NCH) ^ row_swizzle<RB, MF>(r);
            col_a[j] = c;
            voff_a[j] = (r < rows_a) ? (uint32_t)(r * k_bytes + c * 16 + kRsrcBias - (j & 3) * 1024) : kOutOfRange;
        }
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j) {
            const int g = li * B_LOADS + j;
            const int r = g * ROWS_PER_LOAD + lane / NCH;
            const int c = (lane % NCH) ^ row_swizzle<RB, MF>(r);
            col_b[j] = c;
            voff_b[j] = (r < rows_b) ? (uint32_t)(r * k_bytes + c * 16 + kRsrcBias - (j & 3) * 1024) : kOutOfRange;
        }
    }

    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < MM::regs; ++q)
                    acc[i][j][q] = 0.0f;
    }

    // Load q (0 <= q < LOADS) of chunk `chunk` (absolute index along K) into
    // `slot`: q < A_LOADS are A row groups, the rest B row groups.  Every wave
    // issues the same number of loads per chunk, which is what the vmcnt waits
    // count.
    // A load with valid == false reads nothing from memory and fills its LDS
    // block with zeros (it keeps the per-chunk load count uniform).
    // RFL: the descriptors were set up under a branch (the persistent ring
    // re-runs setup() only when its loads move to the next tile), where the
    // compiler cannot keep them in scalar registers by itself; reading them
    // back with readfirstlane does (the LDS-DMA loads take them from scalar
    // registers).
    template <bool RFL = false>
    __device__ __forceinline__ void issue_one(int chunk, int slot, int q, bool valid = true)
    {
        const int64_t kb = (int64_t)chunk * RB;   // byte offset of the chunk in a row
        const int64_t rem = valid ? k_bytes - kb : 0;   // bytes of the row left from kb
        const uint32_t soff = (uint32_t)kb;
        const uint32_t sbase = smem_base + slot * SLOT_BYTES;
        if (q < A_LOADS) {
            const int j = q;
            const uint32_t v = (col_a[j] * 16 < rem) ? voff_a[j] : kOutOfRange;
            const i32x4 r = RFL ? uniform4(rsrc_a) : rsrc_a;
            if ((j & 3) == 0)
                dma16_set_m0(r, sbase + (li * A_LOADS + j) * 1024, v, soff);
            else
                dma16_same_m0(r, j & 3, v, soff);
        } else {
            const int j = q - A_LOADS;
            const uint32_t v = (col_b[j] * 16 < rem) ? voff_b[j] : kOutOfRange;
            const i32x4 r = RFL ? uniform4(rsrc_b) : rsrc_b;
            if ((j & 3) == 0)
                dma16_set_m0(r, sbase + BM * RB + (li * B_LOADS + j) * 1024, v, soff);
            else
                dma16_same_m0(r, j & 3, v, soff);
        }
    }

    __device__ __forceinline__ static i32x4 uniform4(i32x4 x)
    {
        return i32x4{__builtin_amdgcn_readfirstlane(x[0]), __builtin_amdgcn_readfirstlane(x[1]),
                     __builtin_amdgcn_readfirstlane(x[2]), __builtin_amdgcn_readfirstlane(x[3])};
    }

    template <bool RFL = false>
    __device__ __forceinline__ void issue(int chunk, int slot, bool valid = true)
    {
#pragma unroll
        for (int q = 0; q < LOADS; ++q) issue_one<RFL>(chunk, slot, q, valid);
    }

    // Wait until at most j chunks' loads of this wave (j clamped to
    // [0, J]) are still in flight: the chunk issued just before those has
    // landed.  j is uniform; vmcnt takes only immediates, hence the ladder.
    template <int J>
    __device__ __forceinline__ void wait_chunks_after(int j)
    {
        if constexpr (J <= 0) {
            wait_vmcnt<0>();
        } else {
            if (j >= J)
                wait_vmcnt<LOADS * J>();
            else
                wait_chunks_after<J - 1>(j);
        }
    }

    __device__ __forceinline__ void read_one(int slot, int ks, int buf, int r)
    {
        const char *base = smem + slot * SLOT_BYTES;
        const int col = (((kg * KSW + ks) * STEP_COLS + lcol) ^ sw) * 16;
        if (r < FM)
            fa[buf][r] = *reinterpret_cast<const i32x4 *>(base + rd_a + r * FRAG_ROWS * RB + col);
        else
            fb[buf][r - FM] = *reinterpret_cast<const i32x4 *>(base + rd_b + (r - FM) * MF * RB + col);
    }

    __device__ __forceinline__ void mfma_one(int buf, int t)
    {
        const int i = t / FN, j = t % FN;
        acc[i][j] = MM::step(fb[buf][j], fa[buf][i], acc[i][j]);
    }

    // Fragment read r of a k-step for a wave whose first FML fragment rows
    // are live: r < FML reads A fragment r, the rest the FN B fragments (no
    // reads at all when FML == 0).
    template <int FML>
    __device__ __forceinline__ void read_live(int slot, int ks, int buf, int r)
    {
        read_one(slot, ks, buf, r < FML ? r : FM + (r - FML));
    }
    template <int FML>
    static constexpr int reads_live() { return FML > 0 ? FML + FN : 0; }

    // One k-step of chunk i (in `slot`): its MFMAs, interleaved with the
    // fragment reads of the k-step RA ahead (in `next` past the chunk's end)
    // and, in the first SPREAD k-steps, the loads of chunk `load_chunk` into
    // slot `fill`.  Only the MFMAs and reads of fragment rows 0 .. FML - 1;
    // the loads are the same for every FML.
    template <int FML = FM>
    __device__ __forceinline__ void step(int ks, int slot, int next, int fill, int load_chunk, bool valid)
    {
        constexpr int NMFL = FML * FN;
        constexpr int NRDL = reads_live<FML>();
        constexpr int LGAP = (NMFL / LPK) > 0 ? (NMFL / LPK) : 1;    // MFMAs between loads
        const int t = ks + RA;                 // k-step whose fragments are read now
        const bool in_next = t >= KSW;         // ... of the next chunk
        const int tks = in_next ? t - KSW : t;
        const int tbuf = t % NB;
        const int rslot = in_next ? next : slot;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NMFL; ++m) {
            mfma_one(ks % NB, m);
            if (m < NRDL) read_live<FML>(rslot, tks, tbuf, m);
            if (NP == 0 && ks < SPREAD && m % LGAP == 0 && m / LGAP < LPK) {
                const int q = ks * LPK + m / LGAP;
                if (q < LOADS) issue_one(load_chunk, fill, q, valid);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // reads and loads that did not fit between the MFMAs
#pragma unroll
        for (int r = NMFL; r < NRDL; ++r) read_live<FML>(rslot, tks, tbuf, r);
        if (NP == 0 && ks < SPREAD) {
#pragma unroll
            for (int u = (NMFL + LGAP - 1) / LGAP; u < LPK; ++u) {
                const int q = ks * LPK + u;
                if (q < LOADS) issue_one(load_chunk, fill, q, valid);
            }
        }
    }

    // Tile q of the [l][tile] order of a problem -> (batch, tile row, tile column).
    __device__ __forceinline__ static void tile_of(const TileParams &p, int q, int &lq, int &tm, int &tn)
    {
        const int tiles = p.tiles_m * p.tiles_n;
        lq = q / tiles;
        raster(q % tiles, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    }

    // The producer/consumer ring over the whole sequence of this workgroup's
    // tiles (tiles w, w + G, w + 2G, ... of the [l][tile] order, ntiles of
    // them), C = p.total_chunks chunks each: the ring's units are the
    // (tile, chunk) pairs, tile-major, with the slots, waits and barriers of
    // run(), so the first chunks of the next tile are loaded while the MFMA
    // waves finish the current one.  After the barrier that ends a tile's last
    // unit the MFMA waves stage the tile in `stage` (STAGE_BYTES of LDS beside
    // the ring), every wave meets at one more barrier, and the MFMA waves
    // store the staged tile while the producers go on loading.  The staging
    // area is written again only after at least one more unit barrier, which
    // every MFMA wave passes after its stores (hence its reads of the staged
    // tile) have been issued.
    template <int MODE>
    __device__ void run_persistent(const TileParams &p, int w, int G, int ntiles, char *stage)
    {
        static_assert(NP > 0 && P >= 2 && WK == 1, "the persistent ring uses producer waves");
        static_assert(MODE != MODE_PARTIAL, "the persistent grid does not split K");
        static_assert((NWM * 64) % (BN * (int)sizeof(T) / 16) == 0, "MFMA threads store whole rows of the tile");
        const int C = p.total_chunks;
        const int U = ntiles * C;
        if (U <= 0) return;   // the same for every wave of the workgroup
        if (!mma) {
            // setup() runs only when the loads move on to the next tile: it
            // costs a few hundred cycles, which must not delay every chunk's
            // loads
            int loaded = -1;   // tile (0 .. ntiles - 1) whose descriptors are set up
            int lt = 0, lc = 0;   // tile and chunk of the next unit to load
            int fill = 0;
            for (int j = 0; j < P; ++j) {
                if (lt != loaded && lt < ntiles) {
                    int lq, tm, tn;
                    tile_of(p, w + lt * G, lq, tm, tn);
                    setup(p, lq, tm, tn);
                    loaded = lt;
                }
                issue<true>(lc, fill, j < U);
                ++fill;
                if (++lc == C) {
                    lc = 0;
                    ++lt;
                }
            }
            wait_vmcnt<LOADS * (P - 2)>();   // units 0 and 1 have landed
            block_barrier();
            int ci = 0;   // chunk of the unit being consumed
            for (int i = 0; i < U; ++i) {
                if (lt != loaded && lt < ntiles) {
                    int lq, tm, tn;
                    tile_of(p, w + lt * G, lq, tm, tn);
                    setup(p, lq, tm, tn);
                    loaded = lt;
                }
                issue<true>(lc, fill, i + P < U);
                if (++lc == C) {
                    lc = 0;
                    ++lt;
                }
                wait_vmcnt<LOADS * (P - 2)>();
                block_barrier();                       // end of unit i
                if (++ci == C) {
                    ci = 0;
                    lds_barrier();                     // the tile of unit i is staged
                }
                fill = (fill + 1 == SLOTS) ? 0 : fill + 1;
            }
            wait_vmcnt<0>();
        } else {
            T *out = reinterpret_cast<T *>(p.C);
            block_barrier();
#pragma unroll
            for (int ks = 0; ks < RA; ++ks)
#pragma unroll
                for (int r = 0; r < NRD; ++r) read_one(0, ks, ks % NB, r);
            int slot = 0;
            int cidx = 0, tile = 0;   // chunk and tile of unit i
            for (int i = 0; i < U; ++i) {
                if (cidx == 0) zero();
                const int next = (slot + 1 == SLOTS) ? 0 : slot + 1;
#pragma unroll
                for (int ks = 0; ks < KSW; ++ks) step(ks, slot, next, 0, 0, false);
                block_barrier();                       // end of unit i
                if (cidx == C - 1) {
                    int lq, tm, tn;
                    tile_of(p, w + tile * G, lq, tm, tn);
                    m0 = (int64_t)tm * BM;
                    n0 = (int64_t)tn * BN;
                    stage_tile<MODE, T>(stage);
                    lds_barrier();                     // the tile is staged
                    store_from_stage<MODE, T>(stage, out + (int64_t)lq * p.M * p.N, p.M, p.N, NWM * 64,
                                              (int)threadIdx.x);
                }
                if (++cidx == C) {
                    cidx = 0;
                    ++tile;
                }
                slot = next;
            }
        }
    }

    // acc += sum over chunks [c_begin, c_begin + nk) of the tile.  On entry no
    // load of this workgroup is in flight; on exit none is, and every wave is
    // past its last LDS read of the range.  FRESH: the workgroup's first use
    // of the slots (nothing can still be reading them).
    template <bool FRESH = false, int FML = FM>
    __device__ void run(int c_begin, int nk)
    {
        constexpr int NMFL = FML * FN;
        constexpr int NRDL = reads_live<FML>();
        if constexpr (!FRESH) lds_barrier();   // the slots may still be read by a previous range
        if constexpr (P == 0) {
            for (int i = 0; i < nk; ++i) {
                if (i > 0) lds_barrier();   // everyone is done reading the single slot
                issue(c_begin + i, 0);
                wait_vmcnt<0>();
                lds_barrier();              // every wave's part of chunk i has landed
#pragma unroll
                for (int ks = 0; ks < KSW; ++ks) {
#pragma unroll
                    for (int r = 0; r < NRDL; ++r) read_live<FML>(0, ks, ks & 1, r);
#pragma unroll
                    for (int t = 0; t < NMFL; ++t) mfma_one(ks & 1, t);
                }
            }
        } else if constexpr (NP > 0) {
            if (nk <= 0) return;
            if (!mma) {
                // Only real chunks are loaded (no zero fills past the last
                // one: the MFMA waves' reads past the end are never used), so
                // near the end fewer loads follow the chunk waited for.
                if constexpr (WIN_MEET) {
#pragma unroll
                    for (int c = 0; c < SLOTS; ++c)
                        if (c < nk) issue(c_begin + c, c);
                    wait_chunks_after<P>(min(SLOTS, nk) - 1);   // chunk 0 has landed
                    block_barrier();
                    int fill = 0;
                    for (int i = 0; i < nk; ++i) {
                        // chunk i + 1 has landed (chunks up to i + P were issued)
                        wait_chunks_after<P - 1>(min(i + P, nk - 1) - (i + 1));
                        block_barrier();   // k-step WIN of chunk i: slot i is free
                        if (i + SLOTS < nk) issue(c_begin + i + SLOTS, fill);
                        fill = (fill + 1 == SLOTS) ? 0 : fill + 1;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < P; ++c)
                        if (c < nk) issue(c_begin + c, c);
                    wait_chunks_after<P - 2>(min(P, nk) - 2);   // chunks 0 and 1 have landed
                    block_barrier();
                    int fill = P;
                    for (int i = 0; i < nk; ++i) {
                        if (i + P < nk) issue(c_begin + i + P, fill);   // into the slot of chunk i - 1
                        // chunk i + 2 has landed (chunks up to i + P were issued)
                        wait_chunks_after<P - 2>(min(i + P, nk - 1) - (i + 2));
                        block_barrier();   // end of chunk i
                        fill = (fill + 1 == SLOTS) ? 0 : fill + 1;
                    }
                }
                wait_vmcnt<0>();
            } else {
                block_barrier();
#pragma unroll
                for (int ks = 0; ks < RA; ++ks)
#pragma unroll
                    for (int r = 0; r < NRDL; ++r) read_live<FML>(0, ks, ks % NB, r);
                int slot = 0;
                for (int i = 0; i < nk; ++i) {
                    const int next = (slot + 1 == SLOTS) ? 0 : slot + 1;
#pragma unroll
                    for (int ks = 0; ks < KSW; ++ks) {
                        // this wave's reads of slot i are complete; chunk i + 1 is in
                        if (WIN_MEET && ks == WIN) lds_barrier();
                        step<FML>(ks, slot, next, 0, 0, false);
                    }
                    // every MFMA of chunk i is issued, so its reads of slot i have completed
                    if (!WIN_MEET) block_barrier();
                    slot = next;
                }
            }
        } else {
            if (nk <= 0) return;
            // The ring.  During iteration i (consuming chunk i from slot i mod
            // SLOTS) the loads of chunk i + P go to slot (i + P) mod SLOTS, the
            // slot chunk i - 1 used; fragment reads run RA k-steps ahead of
            // their MFMAs, into chunk i + 1 during the last RA k-steps.
            //
            // The loop body has no branches, so that the compiler can count
            // the LDS reads in flight exactly: past the last chunk the loads
            // become zero fills of the free slot (valid == false) and the reads
            // of the chunk after the last one land in registers that are never
            // used.  Every wait sees the same number of loads issued after the
            // chunk it waits for, hence one vmcnt value for every wait.
#pragma unroll
            for (int c = 0; c < P; ++c) issue(c_begin + min(c, nk - 1), c, c < nk);
            // chunks 0 and 1 (P >= 2), or chunk 0 (P == 1), have landed
            wait_vmcnt<LOADS * (P - 1) - (P >= 2 ? LOADS : 0)>();
            lds_barrier();
#pragma unroll
            for (int ks = 0; ks < RA; ++ks)
#pragma unroll
                for (int r = 0; r < NRDL; ++r) read_live<FML>(0, ks, ks % NB, r);
            int slot = 0;
            int fill = P;   // slot that receives chunk i + P
            for (int i = 0; i < nk; ++i) {
                const int next = (slot + 1 == SLOTS) ? 0 : slot + 1;
                const bool valid = i + P < nk;
                const int load_chunk = c_begin + min(i + P, nk - 1);
#pragma unroll
                for (int ks = 0; ks < KSW; ++ks) {
                    if constexpr (P == 1) {
                        if (ks == WIN) {
                            // chunk i + 1 (all its loads were issued before
                            // k-step WIN) has landed
                            wait_vmcnt<0>();
                            lds_barrier();
                        }
                    }
                    step<FML>(ks, slot, next, fill, load_chunk, valid);
                }
                if constexpr (P >= 2) {
                    wait_vmcnt<WAIT_CNT>();
                    block_barrier();
                }
                slot = next;
                fill = (fill + 1 == SLOTS) ? 0 : fill + 1;
            }
            // the zero fills past the last chunk must land before the slots
            // are reused or the workgroup's LDS is released
            wait_vmcnt<0>();
        }
    }

    // run() for a tile whose first `live` rows exist (live <= BM): each MFMA
    // wave computes only its fragment rows that start before row `live`
    // (interleaved rows: every wave row gets its share of the live blocks).
    // The loads, waits and barriers are those of run() for every wave.
    template <bool FRESH = false>
    __device__ void run_live(int c_begin, int nk, int live)
    {
        static_assert(ILV, "row-block skipping shares the live blocks out over the wave rows");
        const int blocks = (live + MF - 1) / MF;                 // live MF-row blocks
        int fml = (blocks - wm + WAVES_M - 1) / WAVES_M;          // ... of this wave row
        fml = fml < 0 ? 0 : (fml > FM ? FM : fml);
        if (!mma) fml = FM;
        run_fml<FRESH, FM>(c_begin, nk, fml);
    }
    template <bool FRESH, int F>
    __device__ __forceinline__ void run_fml(int c_begin, int nk, int fml)
    {
        if constexpr (F <= 0) {
            run<FRESH, 0>(c_begin, nk);
        } else {
            if (fml >= F)
                run<FRESH, F>(c_begin, nk);
            else
                run_fml<FRESH, F - 1>(c_begin, nk, fml);
        }
    }

    // Accumulator registers 4q .. 4q+3 (0 <= q < NREG / 4).
    __device__ __forceinline__ f32x4v get4(int q) const
    {
        constexpr int GR = MM::regs / 4;
        const int i = q / (FN * GR), j = (q / GR) % FN, g = q % GR;
        return f32x4v{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    }
    __device__ __forceinline__ void set4(int q, f32x4v v)
    {
        constexpr int GR = MM::regs / 4;
        const int i = q / (FN * GR), j = (q / GR) % FN, g = q % GR;
        acc[i][j][4 * g] = v[0];
        acc[i][j][4 * g + 1] = v[1];
        acc[i][j][4 * g + 2] = v[2];
        acc[i][j][4 * g + 3] = v[3];
    }

    // Epilogue.  With the operands swapped, fragment (i, j) holds C^T:
    //   MF = 16: value q of lane -> m = lane % 16, n = 4 (lane / 16) + q
    //   MF = 32: value 4 g + q   -> m = lane % 32, n = 8 g + 4 (lane / 32) + q
    // MODE 0..2 store epilogue(acc) rounded to T into C (batch l); MODE_PARTIAL
    // stores the raw fp32 sums into W ([M][N] for this batch and split).
    // WK > 1: the accumulators of k-group 0 become the sum over the groups,
    // added in ascending kg through LDS (groups 1 .. WK - 1 one at a time).
    __device__ __forceinline__ void reduce_k()
    {
        if constexpr (WK > 1) {
            constexpr int NQ = NREG / 4;
            const int wl = wave % NWT;
#pragma unroll 1
            for (int k = 1; k < WK; ++k) {
                lds_barrier();   // the ring (or the previous round) is no longer read
                if (kg == k) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
                        *reinterpret_cast<f32x4v *>(smem + ((wl * NQ + q) * 64 + lane) * 16) = get4(q);
                }
                lds_barrier();
                if (kg == 0) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const f32x4v o = *reinterpret_cast<const f32x4v *>(smem + ((wl * NQ + q) * 64 + lane) * 16);
                        f32x4v v = get4(q);
                        v[0] += o[0];
                        v[1] += o[1];
                        v[2] += o[2];
                        v[3] += o[3];
                        set4(q, v);
                    }
                }
            }
        }
    }

    template <int MODE>
    __device__ __forceinline__ void store(void *out, int64_t M, int64_t N)
    {
        reduce_k();
        typedef typename std::conditional<MODE == MODE_PARTIAL, float, T>::type OT;
        if constexpr (BM * BN * (int)sizeof(OT) <= LDS_BYTES)
            store_staged<MODE, OT>(reinterpret_cast<OT *>(out), M, N);
        else
            store_direct<MODE>(out, M, N);
    }

    // The finished tile (epilogue applied, converted to the output type OT)
    // goes to LDS row-major, each row's 16-byte columns XOR-swizzled by the
    // row index; it is then stored with one 16-byte access per lane, lanes
    // running along rows, so that every store instruction writes whole cache
    // lines instead of 8 bytes in each of 32 rows.
    template <int MODE, class OT>
    __device__ __forceinline__ void store_staged(OT *out, int64_t M, int64_t N)
    {
        static_assert(THREADS >= BN * (int)sizeof(OT) / 16, "one pass covers a whole row of 16-byte columns");
        lds_barrier();   // every wave's ring reads and loads are done
        stage_tile<MODE, OT>(smem);
        lds_barrier();   // the whole tile is in LDS
        store_from_stage<MODE, OT>(smem, out, M, N, THREADS, (int)threadIdx.x);
    }

    // Bytes of one finished tile in the staged layout (output type T).
    static constexpr int STAGE_BYTES = BM * BN * (int)sizeof(T);

    // Physical 16-byte column of logical column c in staged row r (NC columns
    // per row): XOR with the row when NC is a power of two, else a rotation by
    // the row (an XOR could leave the row, e.g. 11 ^ 4 = 15 with NC = 12).
    template <int NC>
    static __device__ __forceinline__ int stage_col(int c, int r)
    {
        if constexpr ((NC & (NC - 1)) == 0)
            return c ^ (r & (NC - 1));
        else
            return (c + r) % NC;
    }

    // The MFMA waves of k-group 0 write the finished tile (epilogue applied,
    // converted to OT) to `stage`, row-major with each row's 16-byte columns
    // XOR-swizzled by the row index.
    template <int MODE, class OT>
    __device__ __forceinline__ void stage_tile(char *stage)
    {
        constexpr int OES = (int)sizeof(OT);
        constexpr int ROWB = BN * OES;          // bytes per tile row
        constexpr int NC = ROWB / 16;           // 16-byte columns per row
        constexpr int GROUPS = MM::regs / 4;
        static_assert(ROWB % 16 == 0, "staged store layout");
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if (kg != 0 || !mma) break;   // (k-group 0 holds the sums)
            const int r = row_block(i) + lrow;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int g = 0; g < GROUPS; ++g) {
                    const int cn = wn * WTN + j * MF + g * 8 + lcol * 4;   // first of 4 columns
                    float y[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float v = acc[i][j][4 * g + q];
                        y[q] = (MODE == MODE_PARTIAL) ? v : apply_epilogue<MODE>(v);
                    }
                    const int byte = cn * OES;
                    char *dst = stage + r * ROWB + ((stage_col<NC>(byte >> 4, r) << 4) | (byte & 15));
                    if constexpr (OES == 4)
                        *reinterpret_cast<f32x4v *>(dst) = f32x4v{y[0], y[1], y[2], y[3]};
                    else
                        Elem<T>::store4(reinterpret_cast<T *>(dst), y[0], y[1], y[2], y[3]);
                }
            }
        }
    }

    // Threads 0 .. nthreads - 1 store the staged tile at (m0, n0) of `out`
    // ([M][N]) with one 16-byte access per lane, lanes running along rows, so
    // that every store instruction writes whole cache lines instead of 8
    // bytes in each of 32 rows.
    template <int MODE, class OT>
    __device__ __forceinline__ void store_from_stage(const char *stage, OT *out, int64_t M, int64_t N, int nthreads,
                                                     int t)
    {
        constexpr int OES = (int)sizeof(OT);
        constexpr int ROWB = BN * OES;
        constexpr int NC = ROWB / 16;
        constexpr int EPC = 16 / OES;           // elements per 16-byte column
        const int rpp = nthreads / NC;          // rows per pass
        const int c = t % NC;
        const bool vec16 = ((N * OES) & 15) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
        // (threads rpp * NC .. nthreads - 1 start at row BM and store nothing)
#pragma unroll
        for (int rr = t < rpp * NC ? t / NC : BM; rr < BM; rr += rpp) {
            const i32x4 v = *reinterpret_cast<const i32x4 *>(stage + rr * ROWB + (stage_col<NC>(c, rr) << 4));
            const int64_t gm = m0 + rr;
            const int64_t gn = n0 + c * EPC;
            if (gm >= M) continue;
            OT *dst = out + gm * N + gn;
            if (vec16 && gn + EPC <= N) {
                // the result is not read again by this kernel: a non-temporal
                // store (measured 16.5 -> 16.0 us on the 512x5632x2048 bf16
                // shape); split-K partials stay cached for the reduction
                if constexpr (MODE == MODE_PARTIAL)
                    *reinterpret_cast<i32x4 *>(dst) = v;
                else
                    __builtin_nontemporal_store(v, reinterpret_cast<i32x4 *>(dst));
            } else {
                OT e[EPC];
                __builtin_memcpy(e, &v, 16);
#pragma unroll
                for (int q = 0; q < EPC; ++q)
                    if (gn + q < N) dst[q] = e[q];
            }
        }
    }

    template <int MODE>
    __device__ __forceinline__ void store_direct(void *out, int64_t M, int64_t N)
    {
        if (kg != 0 || !mma) return;   // (k-group 0 holds the sums)
        const bool vec_ok = (N & 3) == 0;
        constexpr int GROUPS = MM::regs / 4;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t m = m0 + row_block(i) + lrow;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int g = 0; g < GROUPS; ++g) {
                    const int64_t n = n0 + wn * WTN + j * MF + g * 8 + lcol * 4;
                    const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
                    const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                    if constexpr (MODE == MODE_PARTIAL) {
                        float *W = reinterpret_cast<float *>(out) + m * N;
                        if (vec_ok && n + 3 < N) {
                            *reinterpret_cast<f32x4v *>(W + n) = f32x4v{v0, v1, v2, v3};
                        } else {
                            const float v[4] = {v0, v1, v2, v3};
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (n + q < N) W[n + q] = v[q];
                        }
                    } else {
                        T *Cr = reinterpret_cast<T *>(out) + m * N;
                        const float y0 = apply_epilogue<MODE>(v0), y1 = apply_epilogue<MODE>(v1);
                        const float y2 = apply_epilogue<MODE>(v2), y3 = apply_epilogue<MODE>(v3);
                        if (vec_ok && n + 3 < N) {
                            Elem<T>::store4(Cr + n, y0, y1, y2, y3);
                        } else {
                            const float y[4] = {y0, y1, y2, y3};
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (n + q < N) Cr[n + q] = Elem<T>::from_f32(y[q]);
                        }
                    }
                }
            }
        }
    }

    // The accumulators of the MFMA waves as an fp32 tile in register order:
    // group q of 4 floats of MFMA thread t at floats (q * NWM * 64 + t) * 4,
    // so that every store and load is a coalesced 16-byte access.  Default
    // cache policy: the stores complete in this XCD's L2, where a workgroup of
    // the same XCD reads them back (split-K fix-up).
    static constexpr int PARTIAL_FLOATS = NWM * 64 * NREG;

    __device__ __forceinline__ void store_partial_l2(float *W)
    {
        static_assert(WK == 1, "one k-group holds the sums");
        if (!mma) return;
        const __amdgpu_buffer_rsrc_t r = partial_rsrc(W);
#pragma unroll
        for (int q = 0; q < NREG / 4; ++q)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, get4(q)), r,
                                                   (q * NWM * 64 + (int)threadIdx.x) * 16, 0, 0);
    }

    // acc = sum over k = 0 .. S-1, in ascending k from the left, of the fp32
    // tiles at W + k * PARTIAL_FLOATS (register order); tile `mine` (if
    // 0 <= mine < S) is taken from the accumulators themselves, which hold
    // exactly what was stored there.  MFMA waves only.
    // the largest divisor of n that is at most `cap`
    static constexpr int block_of(int n, int cap)
    {
        int b = n < cap ? n : cap;
        while (n % b) --b;
        return b;
    }
    // Register groups of 4 floats combined per batch: a batch holds 8 floats
    // per group beside the accumulators (the running sum and the loaded
    // partial).  With 128 accumulator floats per lane in VGPRs (a 64 x 128
    // wave tile of 8 waves) 16 groups spilled 24 registers and 8 none; with
    // 256 (accumulators in AGPRs) 16 spilled 3 and 8 spilled 160.
    static constexpr int combine_batch() { return block_of(NREG / 4, NREG == 128 ? 8 : 16); }

    __device__ __forceinline__ void combine_l2(const float *W, int S, int mine)
    {
        if (!mma) return;
        constexpr int NQ = NREG / 4;
        constexpr int QB = combine_batch();
        static_assert(NQ % QB == 0, "register blocks");
        const __amdgpu_buffer_rsrc_t r = partial_rsrc(W);
#pragma unroll
        for (int q0 = 0; q0 < NQ; q0 += QB) {
            f32x4v sum[QB];
            for (int k = 0; k < S; ++k) {
                f32x4v v[QB];
                if (k == mine) {
#pragma unroll
                    for (int b = 0; b < QB; ++b) v[b] = get4(q0 + b);
                } else {
#pragma unroll
                    for (int b = 0; b < QB; ++b)
                        v[b] = __builtin_bit_cast(
                            f32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                        r, (k * PARTIAL_FLOATS + ((q0 + b) * NWM * 64 + (int)threadIdx.x) * 4) * 4,
                                        0, 0));
                }
                if (k == 0) {
#pragma unroll
                    for (int b = 0; b < QB; ++b) sum[b] = v[b];
                } else {
#pragma unroll
                    for (int b = 0; b < QB; ++b) {
                        sum[b][0] += v[b][0];
                        sum[b][1] += v[b][1];
                        sum[b][2] += v[b][2];
                        sum[b][3] += v[b][3];
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < QB; ++b) set4(q0 + b, sum[b]);
        }
    }

    // A private fp32 copy of the accumulators (a stream-K partial tile), in
    // register order: group q of 4 floats of thread t at (q * THREADS + t) * 4,
    // so that every store and load is a coalesced 16-byte access.
    __device__ __forceinline__ void save_partial(float *W)
    {
        static_assert(WK == 1 && NP == 0, "stream-K pieces keep one k-group and no producers");
        const __amdgpu_buffer_rsrc_t r = partial_rsrc(W);
#pragma unroll
        for (int q = 0; q < NREG / 4; ++q)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, get4(q)), r,
                                                   (q * THREADS + (int)threadIdx.x) * 16, 0, kCoherent);
    }

    // Replace the accumulators by sum_{k < n} piece_k, added in ascending k
    // from the left; piece `mine` is the accumulators themselves, the others are
    // saved partials (W_k = ws + slot_k * BM * BN).
    __device__ __forceinline__ void combine(const float *ws, const int *slots, int n, int mine)
    {
        // Blocks of QB register groups: all loads of one piece's block are
        // issued before any of them is used, so a piece costs one memory
        // round trip per block, not one per register group.
        constexpr int NQ = NREG / 4;
        constexpr int QB = combine_batch();
        static_assert(NQ % QB == 0, "register blocks");
#pragma unroll
        for (int q0 = 0; q0 < NQ; q0 += QB) {
            f32x4v sum[QB];
            for (int k = 0; k < n; ++k) {
                f32x4v v[QB];
                if (k == mine) {
#pragma unroll
                    for (int b = 0; b < QB; ++b) v[b] = get4(q0 + b);
                } else {
                    const __amdgpu_buffer_rsrc_t r = partial_rsrc(ws + (int64_t)slots[k] * (BM * BN));
#pragma unroll
                    for (int b = 0; b < QB; ++b)
                        v[b] = __builtin_bit_cast(
                            f32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                        r, ((q0 + b) * THREADS + (int)threadIdx.x) * 16, 0, kCoherent));
                }
                if (k == 0) {
#pragma unroll
                    for (int b = 0; b < QB; ++b) sum[b] = v[b];
                } else {
#pragma unroll
                    for (int b = 0; b < QB; ++b) {
                        sum[b][0] += v[b][0];
                        sum[b][1] += v[b][1];
                        sum[b][2] += v[b][2];
                        sum[b][3] += v[b][3];
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < QB; ++b) set4(q0 + b, sum[b]);
        }
    }
};


// Data-parallel / split-K grid: one workgroup per (batch, split, tile).
template <class T, int BM, int BN, int RB, int WAVES_M, int WAVES_N, int MF, int P, int MODE, int WK = 1,
          int NP = 0>
__global__ __launch_bounds__((WAVES_M *WAVES_N *WK + NP) * 64) void gemm_tile_kernel(TileParams p)
{
    typedef TileCore<T, BM, BN, RB, WAVES_M, WAVES_N, MF, P, WK, NP> Core;
    __shared__ __attribute__((aligned(1024))) char smem[Core::LDS_BYTES];
    Core c;
    c.init(smem);

    // The operand pointers and sizes in scalar registers before the first
    // branch: every kernel argument then arrives in one round of loads (the
    // compiler would otherwise sink some of them past the early return).
    asm volatile("" : : "s"(p.A), "s"(p.B), "s"(p.C), "s"(p.M), "s"(p.N), "s"(p.K), "s"(p.L),
                 "s"(p.chunks_per_split), "s"(p.total_chunks));
    int l, s, tm, tn;
    map_workgroup(p.map, blockIdx.x, l, s, tm, tn);
    // (the host's map covers exactly the grid; a workgroup outside it would
    // address memory past the operands)
    if (l >= p.L || s >= p.split || tm >= p.tiles_m || tn >= p.tiles_n) return;

    const int chunk0 = s * p.chunks_per_split;
    int nk = p.total_chunks - chunk0;
    if (nk > p.chunks_per_split) nk = p.chunks_per_split;
    if (nk < 0) nk = 0;

    c.setup(p, l, tm, tn);
    c.zero();
    c.template run<true>(chunk0, nk);
    if constexpr (MODE == MODE_PARTIAL)
        c.template store<MODE>(reinterpret_cast<float *>(p.C) + ((int64_t)s * p.L + l) * p.M * p.N, p.M, p.N);
    else
        c.template store<MODE>(reinterpret_cast<T *>(p.C) + (int64_t)l * p.M * p.N, p.M, p.N);
}

// ------------------------------------------------------------------ grouped GEMM

// Groups of rows over one shared K: group g owns rows [offs[g - 1], offs[g])
// of A ([total_M][K]) and C ([total_M][N]) and its own B[g] ([N][K]):
//   C[rows of g] = epilogue( A[rows of g] * B[g]^T )
// (the variable-M grouped GEMM reached through torch adapters on
// "深入解析 CUTLASS CuTe DSL 的 JIT 函数参数生成机制", section 5).
struct GroupedParams {
    const void *A;
    const void *B;
    void *C;
    const int32_t *offs;   // device, G cumulative row ends
    int32_t G;
    int32_t total_m;
    int64_t N, K;
    int32_t tiles_n;
    int32_t row_tiles;     // row tiles the grid covers (an upper bound on the groups' sum)
    int32_t total_chunks;
    int32_t group_m;       // raster group height inside a group
};

// Row tile `tr` of the concatenation of every group's row tiles -> (group,
// row tile within the group, first row, rows of the group); g = -1 past the
// last tile.  Each wave scans the offsets 64 groups at a time (one lane per
// group, a wave prefix sum of the tile counts), so every wave of the
// workgroup reaches the same answer.  Offsets are clamped to a non-decreasing
// sequence in [0, total_m], so no offsets can address rows outside A or C.
// With tr < 0 nothing is looked up: the scan runs over every group and
// returns the total number of row tiles (g stays -1); with tr >= 0 the
// return value is not meaningful.
template <int BM>
__device__ __forceinline__ int find_group(const GroupedParams &gp, int tr, int &g, int &tm, int &row0, int &rows)
{
    const int lane = threadIdx.x & 63;
    int before = 0;      // row tiles of the groups scanned so far
    int prev_end = 0;    // clamped end of the last group scanned
    g = -1;
    for (int j0 = 0; j0 < gp.G; j0 += 64) {
        const int j = j0 + lane;
        int end = j < gp.G ? gp.offs[j] : 0;
        // running maximum over the block (and the previous blocks): clamped ends
        end = max(min(end, gp.total_m), 0);
        int run = end;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(run, d, 64);
            if (lane >= d) run = max(run, v);
        }
        end = max(run, prev_end);
        int start = __shfl_up(end, 1, 64);
        if (lane == 0) start = prev_end;
        const int nt = j < gp.G ? (end - start + BM - 1) / BM : 0;
        int incl = nt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        const int total = __shfl(incl, 63, 64);
        const int x = tr - before;
        if (tr >= 0 && x < total) {
            const unsigned long long hit = __ballot(nt > 0 && x >= incl - nt && x < incl);
            const int src = __ffsll((long long)hit) - 1;
            g = j0 + src;
            tm = x - __shfl(incl - nt, src, 64);
            row0 = __shfl(start, src, 64);
            rows = __shfl(end - start, src, 64);
            return before + total;
        }
        before += total;
        prev_end = __shfl(end, 63, 64);
    }
    return before;
}

// Up to this many groups every workgroup scans all of them first (at most 8
// wave-wide steps), to spread exactly the tiles that exist over the XCDs.
constexpr int kGroupedExactScan = 512;

template <class T, int BM, int BN, int RB, int WAVES_M, int WAVES_N, int MF, int P, int MODE, int NP>
__global__ __launch_bounds__((WAVES_M *WAVES_N + NP) * 64) void gemm_grouped_kernel(GroupedParams gp)
{
    typedef TileCore<T, BM, BN, RB, WAVES_M, WAVES_N, MF, P, 1, NP, true> Core;
    __shared__ __attribute__((aligned(1024))) char smem[Core::LDS_BYTES];
    // Group-major order: group g owns the R_g * tiles_n consecutive ids after
    // those of groups 0 .. g-1 (R_g = its row tiles), and inside a group the
    // tiles follow the usual raster.  Tiles that share a column block of B[g]
    // then run close together, on one XCD, and no raster group mixes two
    // groups' B.
    // The grid covers an upper bound of the tiles (the offsets live on the
    // device).  With few groups the exact count T is scanned first and XCD x
    // (workgroups b = x, x + 8, ...) takes the x-th of 8 contiguous runs of
    // about T / 8 tiles, so that no XCD is left with the empty ids at the
    // end; otherwise the ids are remapped over the whole grid.
    int t;
    if (gp.G <= kGroupedExactScan) {
        int g0, t0, r0, n0;
        const int total = find_group<BM>(gp, -1, g0, t0, r0, n0) * gp.tiles_n;
        const int x = (int)(blockIdx.x & 7), j = (int)(blockIdx.x >> 3);
        const int q = total >> 3, rem = total & 7;
        if (j >= q + (x < rem ? 1 : 0)) return;   // (the same for every wave)
        t = x * q + min(x, rem) + j;
    } else {
        t = xcd_remap(blockIdx.x, gridDim.x);
    }
    const int v = t / gp.tiles_n;   // the v-th row tile of the concatenated groups
    int g, tv, row0, rows;
    find_group<BM>(gp, v, g, tv, row0, rows);
    if (g < 0) return;   // past the groups' row tiles (the same for every wave)
    const int rg = (rows + BM - 1) / BM;
    const int u = t - (v - tv) * gp.tiles_n;   // id inside the group
    int tm, tn;
    raster(u, rg, gp.tiles_n, gp.group_m, tm, tn);
    Core c;
    c.init(smem);
    TileParams p;
    p.A = reinterpret_cast<const T *>(gp.A) + (int64_t)row0 * gp.K;
    p.B = reinterpret_cast<const T *>(gp.B) + (int64_t)g * gp.N * gp.K;
    p.C = reinterpret_cast<T *>(gp.C) + (int64_t)row0 * gp.N;
    p.M = rows;
    p.N = gp.N;
    p.K = gp.K;
    p.L = 1;
    c.setup(p, 0, tm, (int)tn);
    c.zero();
    // a group's last row tile computes only its row blocks that hold rows
    c.template run_live<true>(0, gp.total_chunks, min(rows - tm * BM, BM));
    c.template store<MODE>(p.C, rows, gp.N);
}

// Persistent grid (producer configurations, split 1): G = gridDim.x
// workgroups, one per compute unit; workgroup w (after the XCD remap) takes
// tiles w, w + G, w + 2G, ... of the [l][tile] order, so each round of G
// concurrent tiles is a contiguous block of the raster, and one ring runs
// across all of its tiles (TileCore::run_persistent).
template <class T, int BM, int BN, int RB, int WAVES_M, int WAVES_N, int MF, int P, int MODE, int NP>
__global__ __launch_bounds__((WAVES_M *WAVES_N + NP) * 64) void gemm_persistent_kernel(TileParams p)
{
    typedef TileCore<T, BM, BN, RB, WAVES_M, WAVES_N, MF, P, 1, NP> Core;
    static_assert(Core::LDS_BYTES + Core::STAGE_BYTES <= 160 * 1024, "ring and staging area in LDS");
    __shared__ __attribute__((aligned(1024))) char smem[Core::LDS_BYTES + Core::STAGE_BYTES];
    Core c;
    c.init(smem);
    const int G = gridDim.x;
    const int w = xcd_remap(blockIdx.x, G);
    const int total = p.tiles_m * p.tiles_n * (int)p.L;
    const int ntiles = w < total ? (total - w + G - 1) / G : 0;
    c.template run_persistent<MODE>(p, w, G, ntiles, smem + Core::LDS_BYTES);
}

// ------------------------------------------------------------------ split-K with an in-kernel fix-up

// The XCD (and so the L2) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id()
{
    uint32_t x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
    return x & 15;
}

// Split-K (split_matmul_k of the compiler page's Tile-IR pass list) whose S
// pieces of a tile are summed inside the GEMM kernel, with no second launch.
//   - Placement: workgroup b runs on XCD b % 8 (the hardware hands workgroup
//     ids to the XCDs round-robin).  Tile v of the [l][tile] order belongs to
//     XCD x = v / per, and its piece s is workgroup ((v % per) * S + s) * 8 + x,
//     so the S pieces of a tile share one XCD's L2, and each XCD's tiles are a
//     contiguous run of the raster (they share operand rows and columns).
//   - Each piece stores its fp32 partial tile (default cache policy: the
//     stores complete in its XCD's L2), waits for them, then adds itself to
//     the tile's counter word with one device-scope atomic: the arrival count
//     in bits 0..7 and, for piece s, its XCD id + 1 in bits 8 + 4 s ..
//     11 + 4 s.  The piece that brings the count to S is the last one: it
//     resets the word to zero for the next call, adds the S partials in
//     ascending s (its own from its registers), applies the epilogue once and
//     stores C.  Nothing ever waits for another workgroup.
//   - The last piece reads a partial through its own L2 only when the word
//     says that piece ran on the same XCD.  Otherwise (not expected on this
//     chip; forced by the host with force_remote, for tests) it recomputes
//     that piece's partial itself over the same chunks in the same order,
//     which gives the same bits.  Results are bitwise reproducible and equal
//     to the split-K grid with the separate reduction (same partials, same
//     order of additions).
// Workgroup b of a fix-up grid -> tile v of the [l][tile] order (returned),
// batch l, piece s, tile row and column.  Past the last tile of an XCD's run
// it returns l = L (no tile): per * 8 >= tiles of all batches.
__host__ __device__ __forceinline__ uint32_t fixup_map(const TileMap &m, int per, uint32_t b, int &l, int &s, int &tm,
                                                       int &tn)
{
    const uint32_t rnd = b >> 3;
    const uint32_t j = fdiv(rnd, m.d_split);
    s = (int)(rnd - j * (uint32_t)m.split);
    const uint32_t v = (b & 7) * (uint32_t)per + j;
    const uint32_t lq = fdiv(v, m.d_tiles);
    raster_map(m, v - lq * (uint32_t)m.tiles, tm, tn);
    l = (int)lq;
    return v;
}

struct FixupParams {
    TileParams t;            // split = S (2..6), chunks_per_split, map (tiles, S, raster)
    float *ws;               // [tiles of all batches][S] partial tiles
    uint32_t *counters;      // one word per tile, kCounterStride words apart, zero between calls
    int32_t per;             // tiles per XCD: ceil(tiles of all batches / 8)
    int32_t force_remote;    // treat every other piece as not visible (recompute)
};

constexpr int kMaxFixupSplit = 6;
// Counter words 128 bytes apart, one per cache line: the atomics of different
// tiles then never queue behind each other on one line (fix-up and stream-K).
constexpr int kCounterStride = 32;

template <class T, int BM, int BN, int RB, int WAVES_M, int WAVES_N, int MF, int P, int MODE, int NP>
__global__ __launch_bounds__((WAVES_M *WAVES_N + NP) * 64) void gemm_fixup_kernel(FixupParams fp)
{
    typedef TileCore<T, BM, BN, RB, WAVES_M, WAVES_N, MF, P, 1, NP> Core;
    static_assert(Core::PARTIAL_FLOATS == BM * BN, "a partial tile holds the whole tile");
    __shared__ __attribute__((aligned(1024))) char smem[Core::LDS_BYTES];
    Core c;
    c.init(smem);
    const TileParams &p = fp.t;
    asm volatile("" : : "s"(p.A), "s"(p.B), "s"(p.C), "s"(p.M), "s"(p.N), "s"(p.K), "s"(p.L),
                 "s"(p.chunks_per_split), "s"(p.total_chunks), "s"(fp.ws), "s"(fp.counters));
    const int S = p.split;
    int l, s, tm, tn;
    const uint32_t v = fixup_map(p.map, fp.per, blockIdx.x, l, s, tm, tn);
    // (workgroups past the last tile of an XCD's run hold no tile)
    if (l >= p.L || tm >= p.tiles_m || tn >= p.tiles_n) return;

    const int cps = p.chunks_per_split;
    const int chunk0 = s * cps;
    const int nk = max(0, min(cps, p.total_chunks - chunk0));
    c.setup(p, (int)l, tm, tn);
    c.zero();
    c.template run<true>(chunk0, nk);

    float *slots = fp.ws + (int64_t)v * S * Core::PARTIAL_FLOATS;
    c.store_partial_l2(slots + (int64_t)s * Core::PARTIAL_FLOATS);
    wait_vmcnt<0>();   // this wave's partial stores have completed in the L2
    __syncthreads();   // ... every wave's
    uint32_t *flag = reinterpret_cast<uint32_t *>(smem);   // (the ring is no longer read)
    if (threadIdx.x == 0) {
        const uint32_t me = xcc_id();
        const uint32_t add = 1u + ((me + 1u) << (8 + 4 * s));
        uint32_t *cnt = fp.counters + (int64_t)v * kCounterStride;
        const uint32_t old = __hip_atomic_fetch_add(cnt, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t f = 0;
        if ((int)(old & 0xffu) == S - 1) {   // the last piece of the tile
            const uint32_t word = old + add;
            uint32_t remote = 0;
            for (int k = 0; k < S; ++k) {
                const uint32_t xk = (word >> (8 + 4 * k)) & 15u;
                if (k != s && (xk != me + 1u || fp.force_remote)) remote |= 1u << k;
            }
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            f = 1u | (remote << 1);
        }
        flag[0] = f;
    }
    __syncthreads();
    const uint32_t f = flag[0];
    if (!(f & 1u)) return;   // another piece finishes the tile
    uint32_t remote = __builtin_amdgcn_readfirstlane(f >> 1);
    const bool recomputed = remote != 0;
    while (remote) {
        // a piece whose partial this L2 cannot see: compute it here
        const int k = __builtin_ctz(remote);
        remote &= remote - 1;
        const int ck = k * cps;
        c.zero();
        c.template run<false>(ck, max(0, min(cps, p.total_chunks - ck)));
        c.store_partial_l2(slots + (int64_t)k * Core::PARTIAL_FLOATS);
        wait_vmcnt<0>();
        __syncthreads();
    }
    // (after a recomputation the registers hold another piece: every partial
    // is read from its slot, this piece's own included)
    c.combine_l2(slots, S, recomputed ? -1 : s);
    c.template store<MODE>(reinterpret_cast<T *>(p.C) + (int64_t)l * p.M * p.N, p.M, p.N);
}

// ------------------------------------------------------------------ stream-K

// The (tile, chunk) units of all tiles, tile-major, are cut into gridDim.x
// contiguous ranges of equal size (+-1), one per workgroup (the persistent
// variant of the data-parallel grid).  A tile whose chunks fall into several
// ranges is summed from the pieces in ascending chunk order by whichever piece
// finishes last: every other piece leaves its fp32 partial in the workspace
// and counts itself in the tile's counter.  Pieces, their order and hence the
// result are fixed by the shape and the grid: bitwise reproducible.
struct StreamKParams {
    TileParams t;
    float *ws;        // 2 * gridDim.x partial tiles of BM * BN floats
    int *counters;    // one per tile (all batches), kCounterStride ints apart, zero between calls
    int64_t units;    // tiles * total_chunks
};

// First unit of range g, and the range holding unit u.
__device__ __forceinline__ int64_t range_start(int64_t U, int g, int G) { return U * g / G; }
__device__ __forceinline__ int range_of(int64_t U, int64_t u, int G) { return (int)(((u + 1) * G - 1) / U); }

template <class T, int BM, int BN, int RB, int WAVES_M, int WAVES_N, int MF, int P, int MODE>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void gemm_streamk_kernel(StreamKParams sp)
{
    typedef TileCore<T, BM, BN, RB, WAVES_M, WAVES_N, MF, P> Core;
    __shared__ __attribute__((aligned(1024))) char smem[Core::LDS_BYTES];
    __shared__ int s_flag;
    Core c;
    c.init(smem);
    const TileParams &p = sp.t;
    const int G = gridDim.x;
    const int g = xcd_remap(blockIdx.x, G);   // neighbouring ranges share an XCD
    const int64_t U = sp.units;
    const int C = p.total_chunks;
    const int tiles = p.tiles_m * p.tiles_n;
    int64_t u = range_start(U, g, G);
    const int64_t u_end = range_start(U, g + 1, G);
    while (u < u_end) {
        const int64_t tg = u / C;              // global tile index (all batches)
        const int c0 = (int)(u % C);
        const int c1 = (int)min((int64_t)C, (int64_t)c0 + (u_end - u));
        const int l = (int)(tg / tiles);
        int tm, tn;
        raster((int)(tg % tiles), p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        c.setup(p, l, tm, tn);
        c.zero();
        c.run(c0, c1 - c0);
        T *Cl = reinterpret_cast<T *>(p.C) + (int64_t)l * p.M * p.N;
        if (c0 == 0 && c1 == C) {
            c.template store<MODE>(Cl, p.M, p.N);
        } else {
            // pieces of this tile: ranges g_first .. g_last, in chunk order
            const int g_first = range_of(U, tg * C, G);
            const int g_last = range_of(U, tg * C + C - 1, G);
            const int n = g_last - g_first + 1;
            const int mine = g - g_first;
            int slots[8];   // a piece spans at most 8 ranges: ranges hold >= C / 8 units
            for (int k = 0; k < n && k < 8; ++k) {
                const int gk = g_first + k;
                // a range's first piece goes to its slot 0, its last to slot 1
                slots[k] = 2 * gk + ((range_start(U, gk, G) / C == tg) ? 0 : 1);
            }
            int *cnt = sp.counters + tg * kCounterStride;
            // the piece that holds chunk 0 is normally the last to finish: if
            // every other piece is already in, it need not save its own
            bool last = false;
            // Protocol: a piece's partial is written through to memory (system
            // scope stores), every store has completed (vmcnt 0) before any
            // thread of the workgroup passes the barrier, and only then is the
            // tile's device-scope counter incremented; the piece that brings
            // the count to n - 1 reads the partials back with system-scope
            // loads, which cannot be served by a stale L2 line.
            if (c0 == 0) {
                if (threadIdx.x == 0)
                    s_flag = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
                __syncthreads();
                last = s_flag;
                __syncthreads();
            }
            if (!last) {
                c.save_partial(sp.ws + (int64_t)slots[mine] * (BM * BN));
                asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
                __syncthreads();
                if (threadIdx.x == 0)
                    s_flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
                __syncthreads();
                last = s_flag;
                __syncthreads();
            }
            if (last) {
                c.combine(sp.ws, slots, n, mine);
                c.template store<MODE>(Cl, p.M, p.N);
                if (threadIdx.x == 0)
                    __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        u += c1 - c0;
    }
}

// ------------------------------------------------------------------ split-K reduction

// C = epilogue( sum_{s=0}^{S-1} W[s] ), summed in ascending s.  Four elements a
// thread when every split's slice stays 16-byte aligned (total % 4 == 0),
// else one.
template <class T, int MODE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ W, T *__restrict__ C,
                                                            int64_t total, int split)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if ((total & 3) == 0) {
        const int64_t nvec = total >> 2;
        for (int64_t v = first; v < nvec; v += stride) {
            f32x4v sum = *reinterpret_cast<const f32x4v *>(W + v * 4);
            for (int s = 1; s < split; ++s) {
                const f32x4v x = *reinterpret_cast<const f32x4v *>(W + (int64_t)s * total + v * 4);
                sum[0] += x[0];
                sum[1] += x[1];
                sum[2] += x[2];
                sum[3] += x[3];
            }
            Elem<T>::store4(C + v * 4, apply_epilogue<MODE>(sum[0]), apply_epilogue<MODE>(sum[1]),
                            apply_epilogue<MODE>(sum[2]), apply_epilogue<MODE>(sum[3]));
        }
    } else {
        for (int64_t e = first; e < total; e += stride) {
            float sum = W[e];
            for (int s = 1; s < split; ++s)
                sum += W[(int64_t)s * total + e];
            C[e] = Elem<T>::from_f32(apply_epilogue<MODE>(sum));
        }
    }
}

// ------------------------------------------------------------------ row repacking

// dst[r][k] = src[r][k] for k < K and 0 for K <= k < Kp, r < rows: copies
// operand rows of any element alignment (a row length or base pointer that is
// not a multiple of 16 bytes) into rows of Kp elements, Kp * sizeof(T) a
// multiple of 16, at a 16-byte aligned dst, so that the tile kernels' 16-byte
// loads apply.  The zeros past K add nothing to any dot product.  One
// workgroup per row (grid-stride), one 16-byte piece of dst per thread.
// A row starts `lead` bytes (0, or 2 for a 16-bit row) past a 4-byte
// boundary: each piece is read as 20 bytes from that boundary (a 16-byte and
// a 4-byte buffer load, dword-aligned) and shifted into place with
// v_alignbyte.  A load that reaches past the operand's last byte, or past
// the descriptor's range (2^31 - 1 bytes from the row's start), would come
// back zeroed by the buffer's range check, valid bytes included, so the
// pieces whose 20 bytes do not all lie inside both (the last one or two of
// the last row) are read element by element instead.  The 4-byte word a row
// starts in lies in the operand's allocation.
template <class T>
__global__ __launch_bounds__(256) void pack_rows_kernel(const T *__restrict__ src, T *__restrict__ dst,
                                                        int64_t rows, int64_t K, int64_t Kp)
{
    constexpr int V = 16 / (int)sizeof(T);   // elements per 16-byte piece
    const int64_t vpr = Kp / V;               // pieces per dst row
    const uintptr_t end = reinterpret_cast<uintptr_t>(src + rows * K);
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const uintptr_t row0 = reinterpret_cast<uintptr_t>(src + r * K);
        const uintptr_t base = row0 & ~(uintptr_t)3;
        const uint32_t lead = (uint32_t)(row0 - base);
        const uint64_t avail = end - base;
        const uint64_t lim = avail < 0x7fffffffu ? avail : 0x7fffffffu;   // the descriptor's range
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), (short)0, (int)lim, 0x00020000);
        T *d = dst + r * Kp;
        const T *s = src + r * K;
        for (int64_t v = threadIdx.x; v < vpr; v += 256) {
            const uint64_t off64 = (uint64_t)v * 16;
            const int off = (int)off64;   // below 2^31 wherever it is used
            const int64_t k0 = v * V;
            i32x4 w;
            if (off64 + 20 <= lim) {
                const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
                const int hi = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 16, 0, 0);
                w = lo;
                if (lead != 0) {
                    w[0] = (int)__builtin_amdgcn_alignbyte((unsigned)lo[1], (unsigned)lo[0], lead);
                    w[1] = (int)__builtin_amdgcn_alignbyte((unsigned)lo[2], (unsigned)lo[1], lead);
                    w[2] = (int)__builtin_amdgcn_alignbyte((unsigned)lo[3], (unsigned)lo[2], lead);
                    w[3] = (int)__builtin_amdgcn_alignbyte((unsigned)hi, (unsigned)lo[3], lead);
                }
            } else {
                T e[V];
#pragma unroll
                for (int q = 0; q < V; ++q) e[q] = (k0 + q < K) ? s[k0 + q] : T(0.0f);
                __builtin_memcpy(&w, e, 16);
            }
            if (k0 + V > K) {   // the row's last piece: zeros past K
                T e[V];
                __builtin_memcpy(e, &w, 16);
#pragma unroll
                for (int q = 0; q < V; ++q)
                    if (k0 + q >= K) e[q] = T(0.0f);
                __builtin_memcpy(&w, e, 16);
            }
            *reinterpret_cast<i32x4 *>(d + k0) = w;
        }
    }
}

// ------------------------------------------------------------------ general kernel

// Any alignment, any K: element-wise bounds-checked loads into LDS (as fp32),
// 64 x 64 output tile, 256 threads, 4 x 4 outputs a thread, fp32 FMA.
template <class T, int MODE>
__global__ __launch_bounds__(256) void gemm_general_kernel(const T *__restrict__ A, const T *__restrict__ B,
                                                           T *__restrict__ C, int64_t M, int64_t N, int64_t K,
                                                           int32_t tiles_m, int32_t tiles_n)
{
    constexpr int TB = 64, KB = 16;
    __shared__ float sa[KB][TB + 1];
    __shared__ float sb[KB][TB + 1];
    int t = blockIdx.x;
    const int tm = t % tiles_m;
    t /= tiles_m;
    const int tn = t % tiles_n;
    const int l = t / tiles_n;
    const int64_t m0 = (int64_t)tm * TB, n0 = (int64_t)tn * TB;
    const T *Ab = A + (int64_t)l * M * K;
    const T *Bb = B + (int64_t)l * N * K;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += KB) {
        for (int e = threadIdx.x; e < TB * KB; e += 256) {
            const int r = e / KB, kk = e % KB;
            const int64_t ma = m0 + r, nb = n0 + r, k = k0 + kk;
            sa[kk][r] = (ma < M && k < K) ? Elem<T>::to_f32(Ab[ma * K + k]) : 0.0f;
            sb[kk][r] = (nb < N && k < K) ? Elem<T>::to_f32(Bb[nb * K + k]) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sa[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sb[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n < N) C[((int64_t)l * M + m) * N + n] = Elem<T>::from_f32(apply_epilogue<MODE>(acc[i][j]));
        }
    }
}

}  // namespace gmk
