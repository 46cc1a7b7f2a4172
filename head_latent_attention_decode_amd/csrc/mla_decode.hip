// MLA decode for MI355X (gfx950): split-KV absorbed-query attention over a
// paged latent cache, plus the LSE merge of the split partials.
//
// What is computed (vLLM API docs, vllm.model_executor.layers.attention.
// mla_attention, module docstring, "Data-Movement Friendly Approach (i.e.
// forward_mqa)"; Model-Optimizer docs, modelopt.torch.kernels.quantization.
// attention.mla, mla_attention_decode): every head of a request attends with
// its 576-wide absorbed query over the request's cached rows cat[kv_c, k_pe];
// the value of a row is its first 512 columns.  Output: out [B, N, 512] and
// the natural-log LSE [B, N].
//
// Design (gfx950, wave64):
//  * One workgroup per (request, KV split, head group).  All heads of the
//    group share every KV tile: a tile of rows is fetched from HBM once,
//    straight into LDS with global_load_lds_dwordx4 (no VGPR staging), and
//    read from LDS by every wave.
//  * QK^T runs on bf16 MFMA as S^T = K . Q^T: the K tile (tokens x 576, read
//    from LDS in its natural row-major layout) is the A operand, the query
//    fragments held in VGPRs are the B operand, so each wave's heads form the
//    N dimension and each K fragment read from LDS serves all of them.
//  * The S^T accumulator layout (head on the lane, tokens in registers) is
//    exactly the B-operand layout PV needs for P^T, so the softmax output
//    feeds PV without any cross-lane movement.  PV runs as O^T = V^T . P^T
//    with V^T read from the same LDS tile by ds_read_b64_tr_b16 (a transposed
//    LDS read), so the value rows are never copied or transposed in memory.
//  * Online softmax in the log2 domain with a lazy running maximum: the
//    accumulators are rescaled only when a tile's maximum exceeds the running
//    one by more than 2^8, which keeps every weight <= 256 and skips almost
//    all rescales.  Row maxima and sums use wavefront lane exchanges.
//  * LDS rows are stored with an XOR swizzle of their 16-byte chunks so that
//    both the MFMA operand reads and the transposed reads avoid bank
//    conflicts; the swizzle is applied by choosing which global chunk each
//    lane fetches, since a direct-to-LDS load writes 64 consecutive slots.
//  * Workgroup ids are remapped so consecutive work items share an XCD (and
//    its L2): the splits of one request then reuse its query from L2.
//  * The split partials (normalised output, LSE) go to a caller workspace and
//    a second kernel merges them; with one split the first kernel writes the
//    bf16 output directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <stdlib.h>

#include "mla_decode.h"

namespace {

constexpr int kD = 576;                 // query / row width (Lkv + R)
constexpr int kDV = 512;                // value / output width (Lkv)
constexpr int kRowBytes = kD * 2;       // a bf16 row
constexpr int kRowChunks = kRowBytes / 16;
constexpr int kSplitUnit = 32;          // split boundaries are multiples of this
// Chunks are at least this long, so a short request fills only the first
// splits and the trailing ones are empty: a chunk's fixed costs (query load,
// partial write, its share of the merge) stay small next to its KV rows.
constexpr int kMinChunk = 2048;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;    // log2 headroom before a rescale

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define AS3(ptr) ((LDS_AS uint8_t *)(ptr))
#define CONST_AS __attribute__((address_space(4)))

// Read-only, wave-uniform data (page table entries, lengths, the fp8 scale)
// is read through the constant address space so that it becomes a scalar
// load: scalar loads are tracked by lgkmcnt, so they never force a wait on
// the vector-memory counter that tracks the tile loads in flight.
template <typename T>
__device__ __forceinline__ T load_uniform(const T *p, long long i)
{
    return ((const CONST_AS T *)p)[i];
}

struct Params {
    const __bf16 *q;            // [B, N, 576]  (N: every query row's heads)
    const uint8_t *cache;       // [num_blocks, P, 576] elements
    const float *cache_scale;   // fp8: one float; bf16: unused
    const int32_t *block_table; // [B, MB]
    const int32_t *seq_lens;    // [B]
    float *part_out;            // [B, N, S, 512]   (split mode)
    float *part_lse;            // [B, N, S]
    __bf16 *out;                // [B, N, 512]      (direct mode, S == 1)
    float *lse;                 // [B, N] or null   (direct mode)
    float scale_log2;           // softmax_scale * log2(e)
    int B, N, S, MB, num_blocks, page_shift, HG;
    // Multi-token decode: a request's QL query rows of NR heads each are its
    // N = QL * NR heads, row-major, so that one workgroup may cover several
    // rows.  Head h belongs to row h / NR; a causal row r sees the request's
    // first L - (QL - 1 - r) tokens, other rows all L.  Single-token decode
    // is QL = 1, NR = N.
    int QL, NR, causal;
};

// XOR swizzle of the 16-byte chunks of LDS row r (rows are 1152 bytes):
// logical chunk c of row r is stored at chunk c ^ swz(r), where swz(r) swaps
// bits 1 and 2 of r & 7.  With gfx950's 64 four-byte banks this makes both
// read patterns of a tile conflict-free (measured with the LDS bank-conflict
// counter on every candidate linear swizzle of the low row bits): the
// ds_read_b128 operand reads of QK^T (16 consecutive rows, one chunk each)
// and the ds_read_b64_tr_b16 transposed reads of PV (16-lane groups reading
// 4 consecutive rows x 32 bytes).  The XOR stays inside an aligned group of 8
// chunks, so it never leaves the 72-chunk row, and it depends on r & 7 only.
__device__ __forceinline__ int swz(int r) { return (r & 1) | ((r & 2) << 1) | ((r & 4) >> 1); }

// Workgroup id -> (request, split, head group).  The hardware deals
// consecutive workgroup ids round-robin over the 8 XCDs.  With S a multiple
// of 32, each request's chunks are dealt over the XCDs in runs of 4;
// otherwise, when the grid is a multiple of 8, each XCD gets a contiguous
// range of work items.
__device__ __forceinline__ void decode_work(const Params &p, int &b, int &s, int &hg)
{
    int i = blockIdx.x;
    const int G = gridDim.x;
    if ((p.S & 31) == 0) {
        // S a multiple of 32: XCD x = i & 7 takes the chunks s of request b
        // with (b + s / 4) mod 8 == x.  A request's chunks are dealt over the
        // XCDs in runs of 4 from its own offset, so requests of ragged lengths
        // load the XCDs evenly: contiguous request ranges per XCD left one XCD
        // 16% above the mean on a uniform [1, 32768] batch.  Runs of 4 keep a
        // request's query and page-table rows in one L2 for a while (runs of
        // one were 8% slower than contiguous ranges, runs of 4 5% faster).  The
        // head groups of a chunk stay adjacent on one XCD, so its KV rows meet
        // in one L2.
        const int x = i & 7, k = i >> 3;
        const int S32 = p.S >> 5;
        hg = k % p.HG;
        const int k2 = k / p.HG;          // ((b * S32 + s / 32) * 4) + s % 4
        const int r = k2 & 3, k3 = k2 >> 2;
        b = k3 / S32;
        s = 32 * (k3 % S32) + 4 * ((x - b) & 7) + r;
        return;
    }
    if ((G & 7) == 0)
        i = (i & 7) * (G >> 3) + (i >> 3);
    hg = i % p.HG;
    const int bs = i / p.HG;
    s = bs % p.S;
    b = bs / p.S;
}

// Request b's length, clamped to [0, the page table's capacity].
__device__ __forceinline__ long long request_len(const Params &p, int b)
{
    const long long cap = (long long)p.MB << p.page_shift;
    const long long L = load_uniform(p.seq_lens, b);
    return L < 0 ? 0 : (L > cap ? cap : L);
}

// Token range [t0, t1) of split s of request b.  The chunk length is
// ceil(L / S) rounded up to kSplitUnit and to at least kMinChunk, a function
// of (L, S) only.
__device__ __forceinline__ void chunk_range(const Params &p, int b, int s, int &t0, int &t1)
{
    const long long L = request_len(p, b);
    const long long per = (L + p.S - 1) / p.S;
    long long C = (per + kSplitUnit - 1) / kSplitUnit * kSplitUnit;
    C = C > kMinChunk ? C : kMinChunk;
    const long long a = (long long)s * C;
    const long long e = a + C;
    t0 = (int)(a < L ? a : L);
    t1 = (int)(e < L ? e : L);
}

// End of head h's tokens inside the chunk [t0, t1) of request b: the chunk
// end, cut at a causal row's own length (t0 when the row has none there).
__device__ __forceinline__ int row_end(const Params &p, int b, int h, int t0, int t1)
{
    if (!p.causal || p.QL == 1)
        return t1;
    const long long Lr = request_len(p, b) - (p.QL - 1 - h / p.NR);
    return Lr <= t0 ? t0 : (Lr < t1 ? (int)Lr : t1);
}

__device__ __forceinline__ int clamp_block(int blk, int num_blocks)
{
    return blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
}

// Wait until at most n vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, the other counters
// left at their maximum so they are not waited on).
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Page-table window of one wave: lane i holds the block id of logical page
// base + i of request b, so a tile's block id is one v_readlane away and the
// tile loop issues no memory access for the page table.  Pages only move
// forward within a split, and the window is refilled (a vector load, waited
// for at once) once every 64 pages.
struct PageWindow {
    int base;         // first logical page held (wave-uniform)
    int ids;          // this lane's entry
};

__device__ __forceinline__ void window_fill(const Params &p, PageWindow &win, int b, int page,
                                            int lane)
{
    win.base = page;
    int idx = page + lane;
    idx = idx < p.MB ? idx : p.MB - 1;
    win.ids = p.block_table[(long long)b * p.MB + idx];
    // Wait here, inside the (rare) refill, so that the compiler sees no
    // pending load where the entry is read: otherwise it waits for every
    // vector-memory operation in flight, tile loads included, before each
    // readlane of the window.
    wait_vmcnt<0>();
}

__device__ __forceinline__ int window_block(const Params &p, PageWindow &win, int b, int page,
                                            int lane)
{
    if (page - win.base >= 64)
        window_fill(p, win, b, page, lane);
    return clamp_block(__builtin_amdgcn_readlane(win.ids, page - win.base), p.num_blocks);
}

// One direct-to-LDS load: lane i's 16 bytes at `src` land at LDS byte
// address dst + 16 * i (dst is wave-uniform and goes to M0).  Issued as
// inline assembly so the compiler does not track it: the compiler cannot tell
// which LDS stage a load targets and would otherwise wait for every load in
// flight before each LDS read.  Completion is awaited explicitly with
// wait_vmcnt; the kernels issue no other vector-memory operations while
// tiles are in flight.  The load is nontemporal (nt): each KV row is used once
// by the workgroup that loads it.  On the 16-head kernel, whose rows no other
// workgroup reads, this took long_context's split kernel from 114 to 102 us
// (one interleaved run); on the role-split kernel's full tiles (dma16s), whose
// rows the other head group's workgroup reads through the same L2, it changed
// nothing measurable, so those keep the default policy.
__device__ __forceinline__ void dma16(const void *src, LDS_AS void *dst)
{
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(m0), "v"(src)
                 : "memory", "m0");
}

__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_convertvector(v, bf16x2);
}

// Workgroup barrier that waits only for this wave's LDS operations
// (lgkmcnt(0): its ds_writes have landed and are visible to the other waves
// after the barrier), not for its vector-memory operations: __syncthreads()
// would also wait for every direct-to-LDS tile load in flight, including the
// prefetched ones.  Tile loads are made visible by an explicit wait_vmcnt
// before the barrier.  The memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void barrier_no_fence()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bool wave_any(bool c)
{
    return __builtin_amdgcn_ballot_w64(c) != 0;
}

// ---------------------------------------------------------------------------
// fp8 (E4M3 "FN") cache support.  Rows are staged in LDS as bytes and widened
// to bf16 before the MFMA reads them; E4M3 -> bf16 is exact (3 mantissa bits,
// exponents inside bf16's range), so the only rounding is the fp32 MFMA
// accumulation.  The per-tensor scale is folded into the softmax scale and
// into the final normalisation.
// ---------------------------------------------------------------------------
constexpr int kRowBytes8 = kD;                  // an fp8 row: 576 bytes
constexpr int kRowChunks8 = kRowBytes8 / 16;    // 36

// 4 E4M3 bytes (byte 0 first) -> 4 bf16 values packed as two dwords
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(unsigned v)
{
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true);
    return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// ===========================================================================
// 32-token tiles of bf16 rows, swizzled as above, and the probability rows
// [head][token] the split kernels exchange through LDS.
// ===========================================================================
constexpr int kT32 = 32;                        // tokens per tile
constexpr int kStage32 = kT32 * kRowBytes;      // 36864 bytes (bf16 tile)

// Wait until this wave has at most `k` tiles (k = 0, 1, 2) of loads in flight.
template <int n>
__device__ __forceinline__ void wait_k_tiles(int k)
{
    if (k >= 2) wait_vmcnt<2 * n>(); else if (k == 1) wait_vmcnt<n>(); else wait_vmcnt<0>();
}
template <class Cfg>
__device__ __forceinline__ void wait_tiles_dma(int w, int k)
{
    if (Cfg::kDmaHiWaves != 0 && w < Cfg::kDmaHiWaves)
        wait_k_tiles<Cfg::kDmaLo + 1>(k);
    else
        wait_k_tiles<Cfg::kDmaLo>(k);
}


// ===========================================================================
// Role-split kernel (N a multiple of 64): 64 heads per workgroup, 8 waves,
// two per SIMD.
//   score waves 0..3: wave q scores heads 16q .. 16q+15 (QK^T on
//     v_mfma_f32_16x16x32_bf16 as S^T = K . Q^T, 72 VGPRs of query) and runs
//     the online softmax; it writes bf16 probabilities P[head][token] and the
//     rescale factor of each head to LDS.
//   value waves 4..7: wave v accumulates all 64 heads over output columns
//     128v .. 128v+127 (O^T = V^T . P^T on v_mfma_f32_32x32x16_bf16, 128
//     accumulator registers), reading V^T from the same LDS tile with
//     ds_read_b64_tr_b16.
// Iteration i of the main loop holds one barrier; after it the score waves
// work on tile i while the value waves work on tile i-1, so on every SIMD the
// softmax and LDS traffic of one wave overlap the MFMAs of the other.  Tiles
// are 32 tokens in a 4-stage LDS ring, loaded direct-to-LDS two tiles ahead
// by the value waves.
//   bf16 cache: rows of 1152 bytes.
//   fp8 cache: the E4M3 bytes themselves (rows of 576 bytes in the first half
//     of each stage, half the load instructions); the score waves widen their
//     K fragments and the value waves their V^T fragments to bf16 in
//     registers just before the MFMAs.  The per-tensor scale is folded into
//     the softmax scale and into the final normalisation.
// ===========================================================================
// Tile geometry of the role-split kernel: bf16 tiles are 32 tokens (36,864
// bytes) in a 4-stage ring; fp8 tiles are 64 tokens of E4M3 bytes (the same
// 36,864 bytes) in a 3-stage ring, which leaves room for the longer
// probability rows.  A stage is free again once the barrier after its last
// reader has passed; tiles are loaded two ahead.
template <bool kFp8>
struct WsGeom {
    static constexpr int kTok = kFp8 ? 64 : 32;              // tokens per tile
    static constexpr int kBlocks = kTok / 16;                 // 16-token blocks per tile
    static constexpr int kStages = kFp8 ? 3 : 4;
    static constexpr int kPRow = 2 * kTok + 16;               // bytes per head's P row (+pad)
    static constexpr int kPBytes = 64 * kPRow;                // P of one tile
    static constexpr int kPbuf = kStages * kStage32;          // 2 P buffers
    static constexpr int kAbuf = kPbuf + 2 * kPBytes;         // alpha [2][64]
    static constexpr int kMbuf = kAbuf + 2 * 64 * 4;          // m [64], l [64]
    static constexpr int kLds = kMbuf + 2 * 64 * 4;
    static_assert(kLds <= 160 * 1024, "LDS budget");
    __device__ __forceinline__ static LDS_AS uint8_t *stage(LDS_AS uint8_t *lds, int t)
    {
        return lds + (t % kStages) * kStage32;
    }
};

// Who loads the tiles (each load instruction stalls its wave for tens of
// cycles, so where they go was set by measurement): the 4 value waves, right
// after the barrier, with direct-to-LDS loads of 16 bytes per lane.  A tile
// takes 36 load instructions in either format (32 bf16 rows, or 64 rows of
// E4M3 bytes, widened later at the operand reads), value wave v issuing
// i = v + 4m (m < 9).  Giving the score waves a share made every placement
// slower.
struct WsDma {
    static constexpr int kDmaLo = 9;
    static constexpr int kDmaHiWaves = 0;
};

// One direct-to-LDS load with a wave-uniform 64-bit base in SGPRs and a
// 32-bit per-lane byte offset (the saddr form: no per-lane 64-bit address
// arithmetic).
__device__ __forceinline__ void dma16s(const uint8_t *sbase, int voff, LDS_AS void *dst)
{
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

// fp8 tiles keep their E4M3 bytes in LDS: 32 rows of 576 bytes in the first
// half of a stage, 16-byte chunk c of row r stored at chunk c ^ swz8(r).  The
// score waves read 8 bytes of one row per lane (16 rows of one chunk per
// half-wave) and the value waves read V^T with ds_read_b64_tr_b8 (8 rows of
// one chunk per 16 lanes); with the swizzle both land on distinct banks.
__device__ __forceinline__ int swz8(int r)
{
    // bit 1 from bit 2 of the row and bit 0 from bit 3: rows 4 apart differ in
    // bit 1, so the two 16-lane groups of a transposed read (adjacent chunks
    // of the same 8 rows) never share a bank
    return ((r >> 1) & 2) | ((r >> 3) & 1);
}

// A value wave's tile loads.  Load instruction i fills LDS chunks
// [64i, 64i+64) of the tile: chunk q = 64i + lane is row r = q / kChunks,
// stored position q % kChunks, which holds logical chunk (q % kChunks) ^
// swizzle(r) of the row.  An instruction's rows lie in one 16-row block
// (rows 16h .. 16h+15, h = i / kHalf), hence in one page; per-lane source
// offsets are relative to the block's first row and do not depend on the
// tile.
template <bool kFp8>
struct WsLoader {
    using G = WsGeom<kFp8>;
    static constexpr int kRow = kFp8 ? kRowBytes8 : kRowBytes;
    static constexpr int kChunks = kRow / 16;
    static constexpr int kLoads = G::kTok * kChunks / 64;  // 36 for either format
    static constexpr int kHalf = kLoads / G::kBlocks;      // loads per 16 rows
    static constexpr int kPerWave = (kLoads + 3) / 4;      // 9
    PageWindow win;
    int off[kPerWave];
    int w, lane, b, t_begin, t_end;

    __device__ __forceinline__ static int sw(int r) { return kFp8 ? swz8(r) : swz(r); }

    __device__ __forceinline__ void init(const Params &p, int w_, int lane_, int b_, int t0,
                                         int t1)
    {
        w = w_;
        lane = lane_;
        b = b_;
        t_begin = t0;
        t_end = t1;
#pragma unroll
        for (int m = 0; m < kPerWave; ++m) {
            int i = w + 4 * m;
            i = i < kLoads ? i : w;            // (a slot the wave never issues)
            const int q = i * 64 + lane;
            const int r = q / kChunks;
            const int c = (q % kChunks) ^ sw(r);
            off[m] = (r - 16 * (i / kHalf)) * kRow + c * 16;
        }
        window_fill(p, win, b, t_begin >> p.page_shift, lane);
    }
    // tile t into its stage; rows past t_end repeat row t_end - 1 (finite
    // values whose scores are masked)
    __device__ __forceinline__ void issue(const Params &p, LDS_AS uint8_t *lds, int t)
    {
        const int ts = t_begin + t * G::kTok;
        LDS_AS uint8_t *stage = G::stage(lds, t);
        const int pmask = (1 << p.page_shift) - 1;
        const uint8_t *base[G::kBlocks];
        if (ts + G::kTok <= t_end) {
#pragma unroll
            for (int h = 0; h < G::kBlocks; ++h) {
                const int first = ts + 16 * h;
                const int blk = window_block(p, win, b, first >> p.page_shift, lane);
                base[h] = p.cache + (((long long)blk << p.page_shift) + (first & pmask)) * kRow;
            }
#pragma unroll
            for (int m = 0; m < kPerWave; ++m) {
                const int i = w + 4 * m;
                if (i < kLoads)
                    dma16s(base[i / kHalf], off[m], stage + i * 1024);
            }
        } else {
            const int last = t_end - 1;
#pragma unroll
            for (int h = 0; h < G::kBlocks; ++h) {
                int first = ts + 16 * h;
                first = first < last ? first : last;
                const int blk = window_block(p, win, b, first >> p.page_shift, lane);
                base[h] = p.cache + ((long long)blk << p.page_shift) * kRow;
            }
#pragma unroll
            for (int m = 0; m < kPerWave; ++m) {
                const int i = w + 4 * m;
                if (i < kLoads) {
                    const int q = i * 64 + lane;
                    const int r = q / kChunks;
                    int tok = ts + r;
                    tok = tok < last ? tok : last;
                    const int c = (q % kChunks) ^ sw(r);
                    dma16(base[i / kHalf] + (long long)(tok & pmask) * kRow + c * 16,
                          stage + i * 1024);
                }
            }
        }
    }
    // before the first barrier: tiles 0 and 1
    __device__ __forceinline__ void prologue(const Params &p, LDS_AS uint8_t *lds, int ntiles)
    {
#pragma unroll
        for (int t = 0; t < 2; ++t)
            if (t < ntiles)
                issue(p, lds, t);
    }
    // top of iteration i: this wave's loads of tile i have landed
    __device__ __forceinline__ void before_barrier(int i, int ntiles)
    {
        if (i < ntiles)
            wait_tiles_dma<WsDma>(w, i + 1 < ntiles ? 1 : 0);
    }
    // iteration i: tile i+2 into its stage, last read in iteration i-2 (4
    // stages) or i-1 (3 stages: the score waves' K and the value waves' V^T
    // prefetch of tile i-1, both before this iteration's barrier)
    __device__ __forceinline__ void step(const Params &p, LDS_AS uint8_t *lds, int i, int ntiles)
    {
        if (i + 2 < ntiles)
            issue(p, lds, i + 2);
    }
};

// Eight E4M3 codes widened to bf16 (exact: every E4M3 value is a bf16).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(u32x2 v)
{
    const u32x2 lo = e4m3x4_to_bf16x4(v[0]);
    const u32x2 hi = e4m3x4_to_bf16x4(v[1]);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Scores of one tile (32 bf16 or 64 fp8 tokens) for a score wave's 16 heads,
// lazy online softmax, probabilities and rescale factor to LDS.  MFMA j takes
// K step k = j / NB (32 dimensions) of token block tb = j % NB (16 tokens);
// accumulator j & 3 is tb (NB = 4) or tb + 2 (k & 1) (NB = 2, summed after).
template <bool kMask, bool kFp8>
__device__ __forceinline__ void ws_score_tile(float &m, float &l, const bf16x8 (&qf)[18],
                                              const LDS_AS uint8_t *stage, LDS_AS uint8_t *prow,
                                              LDS_AS float *arow, const int (&ko)[2], int g4,
                                              float scale_log2, int tile_start, int t_end)
{
    constexpr int kAhead = 8;
    constexpr int NB = WsGeom<kFp8>::kBlocks, kMfma = 18 * NB;
    // bf16: 16 bytes of a row; fp8: 8 bytes of a row (codes, widened at the MFMA)
    using Frag = typename std::conditional<kFp8, u32x2, bf16x8>::type;
    auto kfrag = [&](int j) {
        const int k = j / NB, tb = j % NB;
        if constexpr (kFp8)
            return *(const LDS_AS u32x2 *)(stage + ko[k & 1] + (k >> 1) * 64 +
                                           tb * 16 * kRowBytes8);
        else
            return *(const LDS_AS bf16x8 *)(stage + ko[k & 1] + (k >> 1) * 128 +
                                            tb * 16 * kRowBytes);
    };
    f32x4 sc4[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
    Frag kb[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
        kb[j] = kfrag(j);
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int j = 0; j < kMfma; ++j) {
        bf16x8 a;
        if constexpr (kFp8)
            a = e4m3x8_to_bf16x8(kb[j % kAhead]);
        else
            a = kb[j % kAhead];
        if (j + kAhead < kMfma)
            kb[j % kAhead] = kfrag(j + kAhead);
        sc4[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[j / NB], sc4[j & 3], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (j + kAhead < kMfma)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    f32x4 sc[NB];
    if constexpr (NB == 2) {
        sc[0] = sc4[0] + sc4[2];
        sc[1] = sc4[1] + sc4[3];
    } else {
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
            sc[tb] = sc4[tb];
    }
    float x[4 * NB];
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = sc[tb][i] * scale_log2;
            if (kMask) {
                const int tok = tile_start + 16 * tb + 4 * g4 + i;
                x[4 * tb + i] = tok < t_end ? v : -INFINITY;
            } else {
                x[4 * tb + i] = v;
            }
            mx = fmaxf(mx, x[4 * tb + i]);
        }
    float alpha = 1.0f;
    if (wave_any(mx > m + kLazyRescale)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx);
        alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        l *= alpha;
    }
    // The row sum takes the fp32 probabilities, the MFMA their bf16
    // roundings: the LSE stays accurate to fp32 whatever the running maximum.
    // A head that has seen no token yet (a causal row with none in this
    // chunk) keeps m = -inf and gets zero probabilities.
    const float mu = m == -INFINITY ? 0.f : m;
    float lsum = 0.f;
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            e[j] = __builtin_amdgcn_exp2f(x[4 * tb + j] - mu);
        lsum += (e[0] + e[1]) + (e[2] + e[3]);
        const bf16x2 p01 = to_bf16x2(e[0], e[1]);
        const bf16x2 p23 = to_bf16x2(e[2], e[3]);
        *(LDS_AS bf16x4 *)(prow + (16 * tb + 4 * g4) * 2) = bf16x4{p01[0], p01[1], p23[0], p23[1]};
    }
    l += lsum;
    if (g4 == 0)
        *arow = alpha;
}

// V^T fragment j (0..7) of a tile for a value wave: two transposed reads
// giving tokens 16kk + 8 g2 .. +8 of column 128vq + 32cb + r32 (j = cb + 4kk),
// the A operand of O^T = V^T . P^T for both head blocks.
__device__ __forceinline__ bf16x8 ws_vfrag(const LDS_AS uint8_t *stage, const int (&to)[2][2],
                                           int j)
{
    const int cb = j & 3, kk = j >> 2;
    const int off = kk * 16 * kRowBytes + (cb >> 1) * 128;
    const bf16x4 lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(stage + to[0][cb & 1] + off));
    const bf16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(stage + to[1][cb & 1] + off));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// fp8: V^T fragment j of a tile as E4M3 codes, one ds_read_b64_tr_b8: lane
// (G, jj) of 16-lane group G addresses token row 16kk + 8(G >> 1) + (jj >> 1),
// byte 8(jj & 1) of the 16-byte chunk of columns 128vq + 32cb + 16(G & 1);
// the transpose leaves it column jj of that chunk at 8 consecutive tokens.
__device__ __forceinline__ u32x2 ws_vfrag8(const LDS_AS uint8_t *stage, const int (&to8)[2],
                                           int j)
{
    const int cb = j & 3, kk = j >> 2;
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (LDS_AS v2i *)(stage + to8[cb & 1] + (cb >> 1) * 64 + kk * 16 * kRowBytes8));
    return u32x2{(unsigned)r[0], (unsigned)r[1]};
}

// PV of one 32-token tile for a value wave: O^T[col][head] for its 128
// columns (4 blocks of 32) and the 64 heads (2 blocks of 32).  vt holds the
// tile's V^T fragments, read during the previous iteration; as the MFMAs
// consume them, vt is refilled with the fragments of the tile in stage
// `next` (complete and visible since this iteration's barrier).  The
// probabilities and rescale factors are read together, so the MFMAs wait
// for one LDS round trip.
template <bool kFp8, class VFrag, class VOff>
__device__ __forceinline__ void ws_value_tile(f32x16 (&o)[4][2], VFrag (&vt)[4 * WsGeom<kFp8>::kBlocks],
                                              const LDS_AS uint8_t *next,
                                              const LDS_AS uint8_t *pbuf, const LDS_AS float *abuf,
                                              const VOff &to, int r32, int g2)
{
    using G = WsGeom<kFp8>;
    bf16x8 pf[2][G::kBlocks];   // [head block][k-step]: tokens 16kk + 8 g2 .. +8 of head 32hb + r32
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int kk = 0; kk < G::kBlocks; ++kk)
            pf[hb][kk] = *(const LDS_AS bf16x8 *)(pbuf + (32 * hb + r32) * G::kPRow +
                                                  (16 * kk + 8 * g2) * 2);
    const float al0 = abuf[r32], al1 = abuf[32 + r32];
    if (wave_any(al0 != 1.0f || al1 != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            o[cb][0] *= al0;
            o[cb][1] *= al1;
        }
    }
#pragma unroll
    for (int j = 0; j < 4 * G::kBlocks; ++j) {
        bf16x8 a;
        if constexpr (kFp8) {
            a = e4m3x8_to_bf16x8(vt[j]);
            vt[j] = ws_vfrag8(next, to, j);
        } else {
            a = vt[j];
            vt[j] = ws_vfrag(next, to, j);
        }
        const int cb = j & 3, kk = j >> 2;
        o[cb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[0][kk], o[cb][0], 0, 0, 0);
        o[cb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[1][kk], o[cb][1], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
}

// Transposed-read offsets of value wave vq (columns 128vq .. +128): 16-lane
// group G reads token rows 16kk + 8 g2 + 4h + (j >> 2) of columns
// 128vq + 32cb + 16(G & 1) + 4(j & 3) (the A operand of O^T = V^T . P^T).
__device__ __forceinline__ void ws_value_offsets(int vq, int lane, int (&to)[2][2])
{
    const int g2 = lane >> 5, G = lane >> 4, j = lane & 15;
    const int cl = 2 * (G & 1) + ((j >> 1) & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int rr = 4 * h + (j >> 2);
#pragma unroll
        for (int e = 0; e < 2; ++e)
            to[h][e] = (8 * g2 + rr) * kRowBytes + ((4 * e) ^ cl ^ swz(rr)) * 16 + 8 * (j & 1) +
                       256 * vq;
    }
}

// fp8 transposed-read offsets of value wave vq (see ws_vfrag8): to8[e] for
// 32-column blocks cb with cb & 1 == e; the swizzle of a lane's token row
// does not depend on the 16-token step.
__device__ __forceinline__ void ws_value_offsets8(int vq, int lane, int (&to8)[2])
{
    const int G = lane >> 4, jj = lane & 15;
    const int row = 8 * (G >> 1) + (jj >> 1);
    const int sw = swz8(row);
#pragma unroll
    for (int e = 0; e < 2; ++e)
        to8[e] = row * kRowBytes8 + (8 * vq + ((2 * e + (G & 1)) ^ sw)) * 16 + 8 * (jj & 1);
}

// Value-wave epilogue of the role-split kernels: normalise O and write the
// output (direct) or the fp32 partial and lse of each of the 64 heads.
template <bool kDirect>
__device__ __forceinline__ void ws_value_epilogue(const Params &p, const f32x16 (&o)[4][2],
                                                  LDS_AS uint8_t *xr, const LDS_AS float *mbuf,
                                                  long long head0, int s, int vq, int lane,
                                                  float out_scale)
{
    constexpr int kXRow = 528;
    const int r32 = lane & 31, g2 = lane >> 5;
    // The accumulator layout scatters a store instruction over 32 head rows,
    // so the normalised output goes through a wave-private LDS region xr
    // (32 rows of 528 bytes) first, one head block (32 heads x 128 columns)
    // at a time, and leaves as whole row segments: 128 columns of one head,
    // 512 contiguous bytes (fp32 partial) or 256 (bf16 output).  Rows are
    // padded to 528 bytes so the column-block writes spread over the banks.
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const int hh = 32 * hb + r32;
        const float mh = mbuf[hh];
        const float lh = mbuf[64 + hh];
        const float inv = lh > 0.f ? out_scale / lh : 0.f;   // no token: out = 0
        // lane (r32, g2) holds head hh, columns 32cb + 8q4 + 4g2 .. +4
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x16 &a = o[cb][hb];
                *(LDS_AS f32x4 *)(xr + r32 * kXRow + (cb * 32 + q4 * 8 + g2 * 4) * 4) =
                    f32x4{a[4 * q4] * inv, a[4 * q4 + 1] * inv, a[4 * q4 + 2] * inv,
                          a[4 * q4 + 3] * inv};
            }
        const float lse_nat = (mh + __builtin_amdgcn_logf(lh)) * kLn2;
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the region is written
        if (kDirect) {
            // 4 heads per instruction: lane l reads head 4it + (l >> 4),
            // columns 8 (l & 15) .. +8
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int h = 4 * it + (lane >> 4), c = 8 * (lane & 15);
                const f32x4 v0 = *(const LDS_AS f32x4 *)(xr + h * kXRow + c * 4);
                const f32x4 v1 = *(const LDS_AS f32x4 *)(xr + h * kXRow + c * 4 + 16);
                const bf16x2 a0 = to_bf16x2(v0[0], v0[1]), a1 = to_bf16x2(v0[2], v0[3]);
                const bf16x2 a2 = to_bf16x2(v1[0], v1[1]), a3 = to_bf16x2(v1[2], v1[3]);
                *(bf16x8 *)(p.out + (head0 + 32 * hb + h) * kDV + 128 * vq + c) =
                    bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
            }
            if (p.lse && vq == 0 && g2 == 0)
                p.lse[head0 + hh] = lse_nat;
        } else {
            // 2 heads per instruction: lane l reads head 2it + (l >> 5),
            // columns 4 (l & 31) .. +4
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int h = 2 * it + (lane >> 5), c = 4 * (lane & 31);
                *(f32x4 *)(p.part_out + ((head0 + 32 * hb + h) * p.S + s) * kDV + 128 * vq + c) =
                    *(const LDS_AS f32x4 *)(xr + h * kXRow + c * 4);
            }
            if (vq == 0 && g2 == 0)
                p.part_lse[(head0 + hh) * p.S + s] = lse_nat;
        }
        // the reads of this head block are done before the next one
        // overwrites the region
        __builtin_amdgcn_s_waitcnt(0xC07F);
    }
}

template <bool kDirect, bool kFp8>
__global__ __launch_bounds__(512, 1) void mla_split_ws(Params p)
{
    using G = WsGeom<kFp8>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G::kLds];

    int b, s, hg;
    decode_work(p, b, s, hg);
    int t_begin, t_chunk;
    chunk_range(p, b, s, t_begin, t_chunk);
    // the workgroup reads up to its last head's end (a causal row's end grows
    // with the row index); each score wave masks at its own row's end
    const int t_end = row_end(p, b, hg * 64 + 63, t_begin, t_chunk);

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long head0 = (long long)b * p.N + hg * 64;

    if (t_begin >= t_end) {
        // empty split: lse = -inf (its partial output is never read), or, when
        // direct, out = 0 and lse = -inf: each thread clears 64 columns of one head
        const int hh = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 64;
        if (kDirect) {
            __bf16 *o = p.out + (head0 + hh) * kDV + c0;
            for (int cc = 0; cc < 64; cc += 8)
                *(bf16x8 *)(o + cc) = bf16x8{};
            if (p.lse && (threadIdx.x & 7) == 0)
                p.lse[head0 + hh] = -INFINITY;
        } else if ((threadIdx.x & 7) == 0) {
            p.part_lse[(head0 + hh) * p.S + s] = -INFINITY;
        }
        return;
    }

    LDS_AS uint8_t *lds = AS3(smem);
    LDS_AS uint8_t *pbuf = lds + G::kPbuf;
    LDS_AS float *abuf = (LDS_AS float *)(lds + G::kAbuf);
    LDS_AS float *mbuf = (LDS_AS float *)(lds + G::kMbuf);

    const int ntiles = (t_end - t_begin + G::kTok - 1) / G::kTok;
    float scale_log2 = p.scale_log2;
    float out_scale = 1.0f;
    if (kFp8) {
        const float ks = load_uniform(p.cache_scale, 0);
        scale_log2 *= ks;
        out_scale = ks;
    }
    // Each role runs its own copy of the loop (same barriers), so the query
    // registers of the score waves and the accumulators of the value waves
    // are never live at the same time.  Iteration i: after the barrier the
    // loads of tile i are visible (each value wave waited for its own), the
    // value waves are done with tile i-2 (stage (i+2)%4) and with P buffer
    // i%2, and the score waves' P and alpha of tile i-1 are visible.
    if (w < 4) {
        // ---- score wave sq: heads 16sq + r16.  Query fragments qf[k] =
        // q[head][32k + 8 g4 .. +8] (B operand of QK).
        const int r16 = lane & 15, g4 = lane >> 4;
        const int sq = w;
        bf16x8 qf[18];
        const __bf16 *qp = p.q + (head0 + 16 * sq + r16) * kD + g4 * 8;
#pragma unroll
        for (int k = 0; k < 18; ++k)
            qf[k] = *(const bf16x8 *)(qp + 32 * k);
        int ko[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if constexpr (kFp8)
                ko[e] = r16 * kRowBytes8 + ((2 * e + (g4 >> 1)) ^ swz8(r16)) * 16 + 8 * (g4 & 1);
            else
                ko[e] = r16 * kRowBytes + ((4 * e) ^ g4 ^ swz(r16)) * 16;
        }
        LDS_AS uint8_t *prow = pbuf + (16 * sq + r16) * G::kPRow;
        LDS_AS float *arow = abuf + 16 * sq + r16;
        const int t_row = row_end(p, b, hg * 64 + 16 * sq, t_begin, t_chunk);
        float m = -INFINITY, l = 0.f;
        for (int i = 0; i <= ntiles; ++i) {
            barrier_no_fence();
            if (i < ntiles) {
                const int ts = t_begin + i * G::kTok;
                if (ts + G::kTok <= t_row)
                    ws_score_tile<false, kFp8>(m, l, qf, G::stage(lds, i),
                                               prow + (i & 1) * G::kPBytes, arow + (i & 1) * 64,
                                               ko, g4, scale_log2, ts, t_row);
                else
                    ws_score_tile<true, kFp8>(m, l, qf, G::stage(lds, i),
                                              prow + (i & 1) * G::kPBytes, arow + (i & 1) * 64,
                                              ko, g4, scale_log2, ts, t_row);
            }
            if (i == ntiles - 1) {
                // final (m, l) of the wave's heads, read by the value waves
                // after the next barrier
                float lt = l + __shfl_xor(l, 16);
                lt += __shfl_xor(lt, 32);
                if (g4 == 0) {
                    mbuf[16 * sq + r16] = m;
                    mbuf[64 + 16 * sq + r16] = lt;
                }
            }
        }
        return;
    }

    // ---- value wave vq: columns 128vq .. +128 of all 64 heads; it also
    // issues its share of every tile's loads, two tiles ahead.
    // Transposed-read offsets: 16-lane group G reads token rows
    // 16kk + 8 g2 + 4h + (j >> 2) of columns 128vq + 32cb + 16(G & 1) + 4(j & 3)
    // (the A operand of O^T = V^T . P^T).
    const int r32 = lane & 31, g2 = lane >> 5;
    const int vq = w - 4;
    using VOff = typename std::conditional<kFp8, int[2], int[2][2]>::type;
    VOff to;
    if constexpr (kFp8)
        ws_value_offsets8(vq, lane, to);
    else
        ws_value_offsets(vq, lane, to);
    WsLoader<kFp8> ld;
    ld.init(p, vq, lane, b, t_begin, t_end);
    ld.prologue(p, lds, ntiles);
    f32x16 o[4][2];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
        o[cb][0] = o[cb][1] = f32x16{};
    // iteration i: this wave's share of tile i+2's loads, then the PV of
    // tile i-1 with its V^T from registers, reading tile i's V^T for the next
    // iteration (in the last iteration, tile i-1's again: the stage of tile
    // ntiles is the epilogue's)
    typename std::conditional<kFp8, u32x2, bf16x8>::type vt[4 * G::kBlocks];
    for (int i = 0; i <= ntiles; ++i) {
        ld.before_barrier(i, ntiles);
        barrier_no_fence();
        ld.step(p, lds, i, ntiles);
        if (i == 0) {
#pragma unroll
            for (int j = 0; j < 4 * G::kBlocks; ++j) {
                if constexpr (kFp8)
                    vt[j] = ws_vfrag8(lds, to, j);
                else
                    vt[j] = ws_vfrag(lds, to, j);
            }
        } else {
            const int j = i - 1;
            const int nt = i < ntiles ? i : j;
            ws_value_tile<kFp8>(o, vt, G::stage(lds, nt), pbuf + (j & 1) * G::kPBytes,
                                abuf + (j & 1) * 64, to, r32, g2);
        }
    }

    // After the last barrier the value waves read only the stage of tile
    // ntiles-1 and no load is in flight, so the stages of tiles ntiles and
    // ntiles+1 are free (with 3 or 4 stages, both differ from it):
    // value waves 0, 1 take the first, 2, 3 the second.
    ws_value_epilogue<kDirect>(p, o, G::stage(lds, ntiles + (vq >> 1)) + (vq & 1) * 32 * 528,
                               mbuf, head0, s, vq, lane, out_scale);
}

// ===========================================================================
// 16 heads per workgroup: 4 waves, each with its own token stream (16-token
// tiles; the WG's j-th tile goes to wave j % 4) and private LDS, merged
// through LDS at the end.  QK^T on v_mfma_f32_16x16x32_bf16, PV on
// v_mfma_f32_16x16x16_bf16.
//   bf16 cache: 2 bf16 stages per wave (direct-to-LDS loads).
//   fp8 cache: 2 fp8 staging buffers and 1 bf16 stage per wave; the wave
//   widens each staged tile itself just before using it.
// ===========================================================================
constexpr int kT16 = 16;
constexpr int kStage16 = kT16 * kRowBytes;                 // 18432 bytes
constexpr int kStage16f8 = kT16 * kRowBytes8;              // 9216 bytes
constexpr int kWaveLds16 = 2 * kStage16;                   // 36864 bytes per wave
constexpr int kLoadsPerTile16 = kT16 * kRowChunks / 64;    // 18 DMA ops (bf16)
constexpr int kLoadsPerTile16f8 = kT16 * kRowChunks8 / 64; // 9 DMA ops (fp8)

__device__ __forceinline__ void issue_tile16(const Params &p, PageWindow &win,
                                             LDS_AS uint8_t *stage, int lane, int b,
                                             int tile_start, int t_end)
{
    const int last = t_end - 1;
    const int page = tile_start >> p.page_shift;   // 16-aligned tile: one page
    const int blk = window_block(p, win, b, page, lane);
    const int pmask = (1 << p.page_shift) - 1;
    const uint8_t *base = p.cache + ((long long)blk << p.page_shift) * kRowBytes;
#pragma unroll
    for (int j = 0; j < kLoadsPerTile16; ++j) {
        const int q = j * 64 + lane;
        const int r = q / kRowChunks;
        int tok = tile_start + r;
        tok = tok < last ? tok : last;
        const int c = (q % kRowChunks) ^ swz(r);
        dma16(base + (long long)(tok & pmask) * kRowBytes + c * 16, stage + j * 1024);
    }
}

__device__ __forceinline__ void issue_tile16_fp8(const Params &p, PageWindow &win,
                                                 LDS_AS uint8_t *stg, int lane, int b,
                                                 int tile_start, int t_end)
{
    const int last = t_end - 1;
    const int page = tile_start >> p.page_shift;
    const int blk = window_block(p, win, b, page, lane);
    const int pmask = (1 << p.page_shift) - 1;
    const uint8_t *base = p.cache + ((long long)blk << p.page_shift) * kRowBytes8;
#pragma unroll
    for (int j = 0; j < kLoadsPerTile16f8; ++j) {
        const int q = j * 64 + lane;
        const int r = q / kRowChunks8;
        int tok = tile_start + r;
        tok = tok < last ? tok : last;
        dma16(base + (long long)(tok & pmask) * kRowBytes8 + (q % kRowChunks8) * 16,
              stg + j * 1024);
    }
}

// One wave widens its staged fp8 tile (16 rows) into its bf16 stage.
__device__ __forceinline__ void convert_tile16(const LDS_AS uint8_t *stg, LDS_AS uint8_t *stage,
                                               int lane)
{
#pragma unroll
    for (int j = 0; j < kLoadsPerTile16f8; ++j) {
        const int q = j * 64 + lane;
        const int r = q / kRowChunks8, c = q % kRowChunks8;
        const u32x4 v = *(const LDS_AS u32x4 *)(stg + r * kRowBytes8 + c * 16);
        const u32x2 b0 = e4m3x4_to_bf16x4(v[0]), b1 = e4m3x4_to_bf16x4(v[1]);
        const u32x2 b2 = e4m3x4_to_bf16x4(v[2]), b3 = e4m3x4_to_bf16x4(v[3]);
        *(LDS_AS u32x4 *)(stage + r * kRowBytes + ((2 * c) ^ swz(r)) * 16) =
            u32x4{b0[0], b0[1], b1[0], b1[1]};
        *(LDS_AS u32x4 *)(stage + r * kRowBytes + ((2 * c + 1) ^ swz(r)) * 16) =
            u32x4{b2[0], b2[1], b3[0], b3[1]};
    }
}

struct State16 {
    f32x4 o[32];      // O^T accumulators: 32 blocks of 16 output columns
    float m;          // running max (log2), same in the 4 lanes of a head
    float l;          // this lane's share of the row sum
};

__device__ __forceinline__ void compute_tile16(float scale_log2, State16 &st,
                                               const bf16x8 (&qf)[18],
                                               const LDS_AS uint8_t *stage,
                                               const int (&ko)[2], const int (&vo)[4],
                                               int lane, int tile_start, int t_end)
{
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int k = 0; k < 18; k += 2) {
        const bf16x8 a0 = *(const LDS_AS bf16x8 *)(stage + ko[0] + (k >> 1) * 128);
        const bf16x8 a1 = *(const LDS_AS bf16x8 *)(stage + ko[1] + (k >> 1) * 128);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[k], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[k + 1], s1, 0, 0, 0);
    }
    const int g4 = lane >> 4;
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tok = tile_start + g4 * 4 + i;
        const float v = (s0[i] + s1[i]) * scale_log2;
        x[i] = tok < t_end ? v : -INFINITY;
        mx = fmaxf(mx, x[i]);
    }
    if (wave_any(mx > st.m + kLazyRescale)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(st.m, mx);
        const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
        st.m = mnew;
        st.l *= alpha;
#pragma unroll
        for (int c = 0; c < 32; ++c)
            st.o[c] *= alpha;
    }
    const bf16x2 p01 = to_bf16x2(__builtin_amdgcn_exp2f(x[0] - st.m),
                                 __builtin_amdgcn_exp2f(x[1] - st.m));
    const bf16x2 p23 = to_bf16x2(__builtin_amdgcn_exp2f(x[2] - st.m),
                                 __builtin_amdgcn_exp2f(x[3] - st.m));
    st.l += ((float)p01[0] + (float)p01[1]) + ((float)p23[0] + (float)p23[1]);
    const bf16x4 pb = {p01[0], p01[1], p23[0], p23[1]};
    const i16x4 pf = __builtin_bit_cast(i16x4, pb);
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
        const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4 *)(stage + vo[cb & 3] + (cb >> 2) * 128));
        st.o[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), pf,
                                                             st.o[cb], 0, 0, 0);
    }
}

template <bool kDirect, bool kFp8>
__global__ __launch_bounds__(256, 1) void mla_split_h16(Params p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * kWaveLds16];

    int b, s, hg;
    decode_work(p, b, s, hg);
    int t_begin, t_end;
    chunk_range(p, b, s, t_begin, t_end);
    t_end = row_end(p, b, hg * 16, t_begin, t_end);   // the 16 heads share a query row

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const long long row_b0 = (long long)b * p.N + hg * 16;  // first head's row

    if (t_begin >= t_end) {
        // empty split: lse = -inf (its partial output is never read), or, when
        // direct, out = 0 and lse = -inf for 16 heads x 512 columns
        const int hh = threadIdx.x >> 4, c0 = (threadIdx.x & 15) * 32;
        if (kDirect) {
            __bf16 *o = p.out + (row_b0 + hh) * kDV + c0;
            for (int c = 0; c < 32; c += 8)
                *(bf16x8 *)(o + c) = bf16x8{};
            if (p.lse && (threadIdx.x & 15) == 0)
                p.lse[row_b0 + hh] = -INFINITY;
        } else if ((threadIdx.x & 15) == 0) {
            p.part_lse[(row_b0 + hh) * p.S + s] = -INFINITY;
        }
        return;
    }

    // QK A operand: row r16, logical chunk 4k + g4 (even / odd k)
    int ko[2];
    {
        const int f = swz(r16);
#pragma unroll
        for (int e = 0; e < 2; ++e)
            ko[e] = r16 * kRowBytes + ((4 * e) ^ g4 ^ f) * 16;
    }
    // PV transposed reads: group g4 reads token rows 4*g4 .. +3, 16 columns
    int vo[4];
    {
        const int j = lane & 15;
        const int rr = 4 * g4 + (j >> 2);
        const int cl = (j >> 1) & 1;
        const int f = swz(rr);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            vo[m] = rr * kRowBytes + (((2 * m) ^ cl ^ f)) * 16 + 8 * (j & 1);
    }

    float scale_log2 = p.scale_log2;
    float out_scale = 1.0f;
    if (kFp8) {
        const float ks = load_uniform(p.cache_scale, 0);
        scale_log2 *= ks;
        out_scale = ks;
    }

    // query fragments, completed before any tile load is issued so that the
    // explicit vmcnt waits below only ever count tile loads
    bf16x8 qf[18];
    {
        const __bf16 *qrow = p.q + (row_b0 + r16) * kD + g4 * 8;
#pragma unroll
        for (int k = 0; k < 18; ++k)
            qf[k] = *(const bf16x8 *)(qrow + 32 * k);
    }
    PageWindow win;
    window_fill(p, win, b, (t_begin + w * kT16) >> p.page_shift, lane);
    wait_vmcnt<0>();

    State16 st;
#pragma unroll
    for (int c = 0; c < 32; ++c)
        st.o[c] = f32x4{};
    st.m = -INFINITY;
    st.l = 0.f;

    LDS_AS uint8_t *mine_lds = AS3(smem) + w * kWaveLds16;
    const int n16 = (t_end - t_begin + kT16 - 1) / kT16;
    const int mine = n16 > w ? (n16 - w + 3) / 4 : 0;  // tiles w, w+4, ...
    if (!kFp8) {
        LDS_AS uint8_t *sa = mine_lds, *sb = mine_lds + kStage16;
        if (mine > 0)
            issue_tile16(p, win, sa, lane, b, t_begin + w * kT16, t_end);
        for (int i = 0; i < mine; i += 2) {
            const int tA = t_begin + (w + 4 * i) * kT16;
            if (i + 1 < mine) {
                issue_tile16(p, win, sb, lane, b, tA + 4 * kT16, t_end);
                wait_vmcnt<kLoadsPerTile16>();
            } else {
                wait_vmcnt<0>();
            }
            compute_tile16(scale_log2, st, qf, sa, ko, vo, lane, tA, t_end);
            if (i + 1 >= mine)
                break;
            if (i + 2 < mine) {
                issue_tile16(p, win, sa, lane, b, tA + 8 * kT16, t_end);
                wait_vmcnt<kLoadsPerTile16>();
            } else {
                wait_vmcnt<0>();
            }
            compute_tile16(scale_log2, st, qf, sb, ko, vo, lane, tA + 4 * kT16, t_end);
        }
    } else {
        LDS_AS uint8_t *bst = mine_lds;
        LDS_AS uint8_t *stg[2] = {mine_lds + kStage16, mine_lds + kStage16 + kStage16f8};
        if (mine > 0)
            issue_tile16_fp8(p, win, stg[0], lane, b, t_begin + w * kT16, t_end);
        if (mine > 1)
            issue_tile16_fp8(p, win, stg[1], lane, b, t_begin + (w + 4) * kT16, t_end);
        for (int i = 0; i < mine; ++i) {
            if (i + 1 < mine)
                wait_vmcnt<kLoadsPerTile16f8>();
            else
                wait_vmcnt<0>();
            convert_tile16(stg[i & 1], bst, lane);
            if (i + 2 < mine)
                issue_tile16_fp8(p, win, stg[i & 1], lane, b, t_begin + (w + 4 * (i + 2)) * kT16,
                                 t_end);
            compute_tile16(scale_log2, st, qf, bst, ko, vo, lane,
                           t_begin + (w + 4 * i) * kT16, t_end);
        }
    }

    // ---- merge the four waves' states through LDS, in two rounds of 256
    // columns: [4 waves][16 heads][256] floats = 64 KiB, then (m, l).
    float ltot = st.l + __shfl_xor(st.l, 16);
    ltot += __shfl_xor(ltot, 32);
    float *mo = (float *)smem;
    float *ml = (float *)(smem + 65536);          // [4][16 heads][2]: m, l
    const int hh = threadIdx.x >> 4;             // merge: head of this thread
    const int c0 = (threadIdx.x & 15) * 16;      //        16 of the 256 columns
    const long long row = row_b0 + hh;
    float a[4], inv = 0.f, lse_nat = 0.f;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        __syncthreads();
#pragma unroll
        for (int cb = 16 * rr; cb < 16 * rr + 16; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mo[(w * 16 + r16) * 256 + (cb - 16 * rr) * 16 + g4 * 4 + i] = st.o[cb][i];
        if (rr == 0 && g4 == 0) {
            ml[(w * 16 + r16) * 2 + 0] = st.m;
            ml[(w * 16 + r16) * 2 + 1] = ltot;
        }
        __syncthreads();
        if (rr == 0) {
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                M = fmaxf(M, ml[(v * 16 + hh) * 2]);
            float Lsum = 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float mv = ml[(v * 16 + hh) * 2];
                a[v] = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
                Lsum += a[v] * ml[(v * 16 + hh) * 2 + 1];
            }
            inv = out_scale / Lsum;
            lse_nat = (M + __builtin_amdgcn_logf(Lsum)) * kLn2;
        }
#pragma unroll
        for (int c = 0; c < 16; c += 4) {
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc += a[v] * mo[(v * 16 + hh) * 256 + c0 + c + e];
                r[e] = acc * inv;
            }
            const int col = 256 * rr + c0 + c;
            if (kDirect) {
                const bf16x2 v0 = to_bf16x2(r[0], r[1]);
                const bf16x2 v1 = to_bf16x2(r[2], r[3]);
                *(bf16x4 *)(p.out + row * kDV + col) = bf16x4{v0[0], v0[1], v1[0], v1[1]};
            } else {
                *(f32x4 *)(p.part_out + (row * p.S + s) * kDV + col) =
                    f32x4{r[0], r[1], r[2], r[3]};
            }
        }
    }
    if ((threadIdx.x & 15) == 0) {
        if (kDirect) {
            if (p.lse)
                p.lse[row] = lse_nat;
        } else {
            p.part_lse[row * p.S + s] = lse_nat;
        }
    }
}

// ===========================================================================
// LSE merge.  A state with lse = -inf carries no weight and its output is
// not read (an empty chunk leaves it unwritten).
//
// One kernel, templated on the columns each lane owns (kCols = 8, 4, 2 or 1;
// a wave covers 64 * kCols columns, so 512 / (64 * kCols) waves share a
// row).  Few rows take narrow lanes so that enough waves are in flight; many
// rows take wide ones.  Whatever the width, every output element is computed
// the same way: each wave computes its row's total lse with the same lane
// layout (merge_total), and the element is the FMA chain over the row's live
// states in ascending s, starting from 0.  The bits of a row therefore depend
// only on that row's states and S, never on how many rows share the launch.
// ===========================================================================
// Largest state lse of a row and the row's total lse (natural log).
__device__ __forceinline__ void merge_total(const float *ls, int S, int lane, float &M,
                                            float &total)
{
    M = -INFINITY;
    for (int s = lane; s < S; s += 64)
        M = fmaxf(M, ls[s]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        M = fmaxf(M, __shfl_xor(M, d));
    float Z = 0.f;
    if (M != -INFINITY)
        for (int s = lane; s < S; s += 64)
            Z += __builtin_amdgcn_exp2f((ls[s] - M) * kLog2e);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        Z += __shfl_xor(Z, d);
    total = M + __builtin_amdgcn_logf(Z) * kLn2;
}

template <int kCols>
struct MergeVec {
    float v[kCols];
    __device__ __forceinline__ void load(const float *p)
    {
        if constexpr (kCols == 8) {
            const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = a[e];
                v[4 + e] = b[e];
            }
        } else if constexpr (kCols == 4) {
            const f32x4 a = *(const f32x4 *)p;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = a[e];
        } else if constexpr (kCols == 2) {
            const f32x2 a = *(const f32x2 *)p;
            v[0] = a[0];
            v[1] = a[1];
        } else {
            v[0] = *p;
        }
    }
};

// Store kCols values as bf16 (round to nearest even) with one vector store.
template <int kCols>
__device__ __forceinline__ void store_bf16(__bf16 *o, const float (&a)[kCols])
{
    typedef __bf16 vec __attribute__((ext_vector_type(kCols == 1 ? 2 : kCols)));
    if constexpr (kCols == 1) {
        *o = (__bf16)a[0];
    } else {
        vec r;
#pragma unroll
        for (int e = 0; e < kCols; ++e)
            r[e] = (__bf16)a[e];
        *(vec *)o = r;
    }
}

template <int kCols>
__global__ __launch_bounds__(256) void mla_merge(const float *__restrict__ part_out,
                                                 const float *__restrict__ part_lse,
                                                 __bf16 *__restrict__ out,
                                                 float *__restrict__ lse, int rows, int S)
{
    constexpr int kWavesPerRow = kDV / (64 * kCols);
    // states whose values are loaded per round: all of a round's loads are
    // in flight before the first is used
    constexpr int kBatch = 32 / kCols;
    const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long row = wid / kWavesPerRow;
    if (row >= rows)
        return;
    const int cb = (int)(wid % kWavesPerRow);
    const int lane = threadIdx.x & 63;
    const int col = cb * 64 * kCols + lane * kCols;
    const float *ls = part_lse + row * S;
    float M, total;
    merge_total(ls, S, lane, M, total);
    __bf16 *o = out + row * kDV + col;
    float acc[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e)
        acc[e] = 0.f;
    if (M == -INFINITY) {
        store_bf16<kCols>(o, acc);
        if (lse && cb == 0 && lane == 0)
            lse[row] = -INFINITY;
        return;
    }
    const float *po = part_out + row * S * kDV + col;
    for (int c0 = 0; c0 < S; c0 += 64) {
        const float lv = c0 + lane < S ? ls[c0 + lane] : -INFINITY;
        unsigned long long live = __ballot(lv != -INFINITY);
        while (live) {
            int idx[kBatch];
            float wgt[kBatch];
            int n = 0;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (live) {
                    idx[u] = __builtin_ctzll(live);
                    live &= live - 1;
                    const float l = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), idx[u]));
                    wgt[u] = __builtin_amdgcn_exp2f((l - total) * kLog2e);
                    n = u + 1;
                } else {
                    idx[u] = idx[0];   // (loaded, never used)
                    wgt[u] = 0.f;
                }
            }
            MergeVec<kCols> v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                v[u].load(po + (long long)(c0 + idx[u]) * kDV);
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (u < n)
#pragma unroll
                    for (int e = 0; e < kCols; ++e)
                        acc[e] = __builtin_fmaf(wgt[u], v[u].v[e], acc[e]);
        }
    }
    store_bf16<kCols>(o, acc);
    if (lse && cb == 0 && lane == 0)
        lse[row] = total;
}

// ===========================================================================
// Decode-step query concat and cache insert.  One 16-byte chunk per thread:
// first the T * N * 72 chunks of the query (64 from ql_nope, 8 from q_pe per
// (token, head)), then the cache rows: 72 chunks of 8 bf16 each, or for an
// fp8 cache 36 chunks of 16 codes (32 bytes of bf16 input each).
// ===========================================================================
__global__ __launch_bounds__(256) void mla_concat_insert(
    const __bf16 *__restrict__ ql_nope, const __bf16 *__restrict__ q_pe,
    const __bf16 *__restrict__ kv_c, const __bf16 *__restrict__ k_pe,
    const int64_t *__restrict__ slot_mapping, uint8_t *__restrict__ cache,
    __bf16 *__restrict__ q_out, const float *__restrict__ scale_inv, long long nq, int T,
    long long rows, int fp8)
{
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < nq) {
        const long long tn = i / 72;
        const int c = (int)(i % 72);
        const bf16x8 v = c < 64 ? *(const bf16x8 *)(ql_nope + tn * kDV + 8 * c)
                                : *(const bf16x8 *)(q_pe + tn * (kD - kDV) + 8 * (c - 64));
        // every store of this kernel is written once and read by a later one:
        // nontemporal (64 tokens x 128 heads: 4.6 -> 3.9 us; 256 tokens: 12.7 ->
        // 12.9 us)
        __builtin_nontemporal_store(v, (bf16x8 *)(q_out + tn * kD + 8 * c));
        return;
    }
    i -= nq;
    const int per = fp8 ? 36 : 72;
    if (i >= (long long)T * per)
        return;
    const int t = (int)(i / per), c = (int)(i % per);
    const long long slot = slot_mapping[t];
    if (slot < 0 || slot >= rows)
        return;
    if (!fp8) {
        const bf16x8 v = c < 64 ? *(const bf16x8 *)(kv_c + (long long)t * kDV + 8 * c)
                                : *(const bf16x8 *)(k_pe + (long long)t * (kD - kDV) + 8 * (c - 64));
        __builtin_nontemporal_store(v, (bf16x8 *)(cache + (slot * kD + 8 * c) * 2));
        return;
    }
    // 16 elements 16c .. 16c+15 of the row, from kv_c (c < 32) or k_pe
    const __bf16 *src = c < 32 ? kv_c + (long long)t * kDV + 16 * c
                               : k_pe + (long long)t * (kD - kDV) + 16 * (c - 32);
    const bf16x8 a = *(const bf16x8 *)src, b = *(const bf16x8 *)(src + 8);
    const float s = *scale_inv;
    // fp32 product, then saturation to the largest finite E4M3FN magnitude
    // (NaN stays NaN), then the hardware's round-to-nearest-even conversion
    auto q8 = [&](__bf16 x) {
        const float f = (float)x * s;
        return f != f ? f : fminf(fmaxf(f, -448.0f), 448.0f);
    };
    unsigned w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const bf16x8 &h = k < 2 ? a : b;
        const int o = 4 * (k & 1);
        int r = __builtin_amdgcn_cvt_pk_fp8_f32(q8(h[o]), q8(h[o + 1]), 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(q8(h[o + 2]), q8(h[o + 3]), r, true);
        w[k] = (unsigned)r;
    }
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]},
                                (u32x4 *)(cache + slot * kD + 16 * c));
}

// ===========================================================================
// Chunked-context gather: 18 threads per workspace row, each doing the row's
// index chain once (owner, start, page, block) and then moving 4 of its 72
// 16-byte bf16 chunks, or converting 2 of its 36 16-code fp8 chunks (16 codes
// in, 16 bf16 out).  Workspace row i belongs to request token_to_seq[i] and
// holds its token seq_starts[b] + i - cu_seq_lens[b]; indices are clamped so
// that every read stays inside the table and the cache whatever they hold.
// ===========================================================================
__global__ __launch_bounds__(256) void mla_gather(
    const uint8_t *__restrict__ cache, int fp8, const float *__restrict__ scale,
    const int32_t *__restrict__ block_table, int B, int MB, int num_blocks, int page_size,
    const int32_t *__restrict__ cu_seq_lens, const int32_t *__restrict__ token_to_seq,
    const int32_t *__restrict__ seq_starts, __bf16 *__restrict__ dst, long long n_threads)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_threads)
        return;
    const long long tok = i / 18;
    const int k = (int)(i % 18);
    int b = token_to_seq[tok];
    b = b < 0 ? 0 : (b >= B ? B - 1 : b);
    long long pos = (long long)(seq_starts ? seq_starts[b] : 0) + (tok - cu_seq_lens[b]);
    pos = pos < 0 ? 0 : pos;
    long long pg = pos / page_size;
    pg = pg >= MB ? MB - 1 : pg;
    const int blk = clamp_block(block_table[(long long)b * MB + pg], num_blocks);
    const long long row = (long long)blk * page_size + pos % page_size;
    __bf16 *d = dst + tok * kD;
    // Each row is read once and written once: nontemporal loads and stores
    // (dsv3's context, 262144 rows: 123.0 -> 120.1 us; the fp8 path unchanged).
    if (!fp8) {
        const bf16x8 *src = (const bf16x8 *)(cache + row * kD * 2);
        bf16x8 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = __builtin_nontemporal_load(src + k + 18 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_nontemporal_store(v[j], (bf16x8 *)(d + 8 * (k + 18 * j)));
        return;
    }
    // 16 codes at a time, decoded exactly to fp32, times the scale in fp32,
    // rounded to bf16 (nearest even)
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 *src = (const u32x4 *)(cache + row * kD);
    const float sc = *scale;
    u32x4 v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        v[j] = __builtin_nontemporal_load(src + k + 18 * j);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        bf16x8 r[2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[j][w], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[j][w], true);
            const bf16x2 a = to_bf16x2(lo[0] * sc, lo[1] * sc);
            const bf16x2 c = to_bf16x2(hi[0] * sc, hi[1] * sc);
            bf16x8 &o = r[w >> 1];
            const int e = 4 * (w & 1);
            o[e] = a[0];
            o[e + 1] = a[1];
            o[e + 2] = c[0];
            o[e + 3] = c[1];
        }
        __builtin_nontemporal_store(r[0], (bf16x8 *)(d + 16 * (k + 18 * j)));
        __builtin_nontemporal_store(r[1], (bf16x8 *)(d + 16 * (k + 18 * j) + 8));
    }
}

// ===========================================================================
// Two-state merge (the prefill context accumulation): per (token, head) the
// prefix and suffix states combine as out = (wp * p + ws * s) / (wp + ws),
// lse = M + ln(wp + ws), w = e^(lse - M), M the larger lse; two states of
// weight zero give (0, -inf).  One 8-element chunk per thread; the
// D / 8 chunks of a row share a workgroup, so the lse, which may be written
// over its own input, is stored after a workgroup barrier.
// ===========================================================================
__global__ __launch_bounds__(256) void mla_merge_two(
    const __bf16 *prefix_out, const float *prefix_lse, const __bf16 *suffix_out,
    const float *suffix_lse, __bf16 *out, float *out_lse, int T, int N, int D, long long n_chunks)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const int cpr = D / 8;
    const bool live = i < n_chunks;
    const long long rowi = live ? i / cpr : 0;
    const int c = (int)(i % cpr);
    const long long t = rowi / N, n = rowi % N;
    const long long li = n * T + t;
    float lp = -INFINITY, ls = -INFINITY;
    if (live) {
        lp = prefix_lse[li];
        ls = suffix_lse[li];
    }
    const float M = fmaxf(lp, ls);
    float wp = 0.f, ws = 0.f, total = -INFINITY;
    if (live && M != -INFINITY) {
        wp = __builtin_amdgcn_exp2f((lp - M) * kLog2e);
        ws = __builtin_amdgcn_exp2f((ls - M) * kLog2e);
        total = M + __builtin_amdgcn_logf(wp + ws) * kLn2;
        const float inv = 1.0f / (wp + ws);
        wp *= inv;
        ws *= inv;
    }
    // The states are read once and the merged row written once: nontemporal
    // loads and stores (T = 8192, N = 128, D = 128: 137.4 -> 126.7 us).
    if (live) {
        bf16x8 r = bf16x8{};
        if (M != -INFINITY) {
            const bf16x8 p =
                __builtin_nontemporal_load((const bf16x8 *)(prefix_out + rowi * D + 8 * c));
            const bf16x8 q =
                __builtin_nontemporal_load((const bf16x8 *)(suffix_out + rowi * D + 8 * c));
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const bf16x2 v = to_bf16x2(wp * (float)p[e] + ws * (float)q[e],
                                           wp * (float)p[e + 1] + ws * (float)q[e + 1]);
                r[e] = v[0];
                r[e + 1] = v[1];
            }
        }
        __builtin_nontemporal_store(r, (bf16x8 *)(out + rowi * D + 8 * c));
    }
    __syncthreads();
    if (live && c == 0 && out_lse)
        out_lse[li] = total;
}

// ===========================================================================
// Per-head matmuls around the attention: out[b, n, c] = sum_k x[b, n, k] *
// W[n, k, c], the query absorb (K = 128, M = 512, W = W_UK_T) and the output
// up-projection (K = 512, M = 128, W = W_UV).  Both are bound by HBM (a
// weight is used by only B tokens), so a workgroup issues every load it needs
// at once and keeps no loop: 4 waves on one unit (head n, a block of kMb
// columns, a block of 64 batch rows).  The W block (K rows x kMb
// columns) is staged in LDS, rows padded by 16 bytes, and read transposed
// with ds_read_b64_tr_b16 as the A operand of v_mfma_f32_16x16x32_bf16
// computing out^T = W^T . x^T; wave w takes rows 16w .. 16w+15, its x
// fragments (16 bytes per lane and 32-deep k step) loaded straight into
// registers.  The results go back through LDS (over the W block, after a
// barrier) so that every store instruction writes whole output rows.
// Units are numbered head-major and dealt out so that the units of one head
// run back to back on one XCD (workgroup i runs on XCD i mod 8): the W block
// of each row block and the x rows of each column block are re-read from that
// XCD's L2, not from HBM.
// ===========================================================================
template <int K, int kMb>
__global__ __launch_bounds__(256) void mla_head_mm(const __bf16 *__restrict__ x, long long xs_tok,
                                                   long long xs_head, const __bf16 *__restrict__ w,
                                                   __bf16 *__restrict__ out, int B, int N, int M)
{
    constexpr int kRow = kMb * 2 + 16;          // padded LDS row (W block and results)
    constexpr int kSteps = K / 32;              // k steps of one MFMA
    constexpr int kCt = kMb / 16;               // 16-column output tiles
    constexpr int kChunks = kMb / 8;            // 16-byte chunks per W or output row
    constexpr int kRowsPerLd = 256 / kChunks;   // W rows one load instruction covers
    constexpr int kWLd = K / kRowsPerLd;        // W loads per thread
    constexpr int kRowsPerSt = 64 / kChunks;    // output rows one store instruction covers
    static_assert(K % kRowsPerLd == 0 && kMb % 16 == 0 && 64 % kChunks == 0, "tiling");
    static_assert(64 <= K && 16 % kRowsPerSt == 0, "the result tiles fit over the W block");
    __shared__ __attribute__((aligned(16))) uint8_t smem[K * kRow];
    LDS_AS uint8_t *lds = AS3(smem);
    const int nblk = M / kMb, nrb = (B + 63) / 64;
    const unsigned U = (unsigned)N * (unsigned)nblk * (unsigned)nrb;
    const unsigned i = blockIdx.x;
    const unsigned u = (U & 7) ? i : (i & 7) * (U >> 3) + (i >> 3);
    const int rb = (int)(u % (unsigned)nrb);
    const int cb = (int)((u / (unsigned)nrb) % (unsigned)nblk);
    const int n = (int)(u / (unsigned)nrb / (unsigned)nblk);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, kq = lane >> 4;
    const int wrow0 = rb * 64 + wave * 16;      // first batch row of this wave
    // W block: thread t loads chunk t % kChunks of rows t / kChunks + kRowsPerLd * m
    const int wrow = tid / kChunks, wchunk = tid % kChunks;
    const __bf16 *wn = w + (long long)n * K * M + (long long)cb * kMb + 8 * wchunk;
    bf16x8 wv[kWLd];
#pragma unroll
    for (int m = 0; m < kWLd; ++m)
        wv[m] = *(const bf16x8 *)(wn + (long long)(wrow + kRowsPerLd * m) * M);
    // x fragments of this wave's rows (rows past the batch read the last row
    // and are not stored)
    bf16x8 xf[kSteps];
    const __bf16 *xr = x + (long long)min(wrow0 + j, B - 1) * xs_tok + (long long)n * xs_head + 8 * kq;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
        xf[ks] = *(const bf16x8 *)(xr + 32 * ks);
#pragma unroll
    for (int m = 0; m < kWLd; ++m)
        *(LDS_AS bf16x8 *)(lds + (wrow + kRowsPerLd * m) * kRow + 16 * wchunk) = wv[m];
    __syncthreads();
    // (a wave whose rows all lie past the batch computes on the clamped row
    // and stores nothing: an early exit here would let the compiler sink the
    // x loads below the barrier, after the W block has arrived)
    // lane j of group kq reads rows 8kq + 4h + (j >> 2), columns 4(j & 3) .. +4
    // of a 16-column tile and then holds column j at 4 consecutive rows
    int toff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        toff[h] = (8 * kq + 4 * h + (j >> 2)) * kRow + 8 * (j & 3);
    f32x4 acc[kCt];
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
        acc[ct] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (LDS_AS bf16x4 *)(lds + toff[0] + ks * 32 * kRow + ct * 32));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (LDS_AS bf16x4 *)(lds + toff[1] + ks * 32 * kRow + ct * 32));
            const bf16x8 a = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xf[ks], acc[ct], 0, 0, 0);
        }
    }
    // lane (j, kq) holds row j, columns 16ct + 4kq .. +4: write the wave's
    // rows into its own slice of the (now unused) W block, then store whole rows
    __syncthreads();
    LDS_AS uint8_t *tile = lds + wave * 16 * kRow;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
        const bf16x2 p01 = to_bf16x2(acc[ct][0], acc[ct][1]);
        const bf16x2 p23 = to_bf16x2(acc[ct][2], acc[ct][3]);
        *(LDS_AS bf16x4 *)(tile + j * kRow + (16 * ct + 4 * kq) * 2) =
            bf16x4{p01[0], p01[1], p23[0], p23[1]};
    }
    const int sr = lane / kChunks, sc = lane % kChunks;
#pragma unroll
    for (int s = 0; s < 16 / kRowsPerSt; ++s) {
        const int r = s * kRowsPerSt + sr;
        const bf16x8 v = *(const LDS_AS bf16x8 *)(tile + r * kRow + 16 * sc);
        if (wrow0 + r < B)
            // written once and read by a later kernel: a nontemporal store
            // (absorb at B = 64, N = 128: 6.5 -> 5.8 us; B = 256: 13.9 -> 13.0 us)
            __builtin_nontemporal_store(
                v, (bf16x8 *)(out + ((long long)(wrow0 + r) * N + n) * M + (long long)cb * kMb +
                              8 * sc));
    }
}

// ===========================================================================
// Device-side check of the decode's data preconditions (seq_lens in range,
// the pages a request uses in [0, num_blocks)), which the decode kernels do
// not check: they clamp instead.  One workgroup of 16 waves; wave w checks
// requests w, w + 16, ..., its lanes spread over the request's table entries.
// The findings meet in LDS and one thread writes the 3-word status.
// ===========================================================================
__global__ __launch_bounds__(1024) void mla_check(const int32_t *__restrict__ block_table,
                                                  const int32_t *__restrict__ seq_lens, int B,
                                                  int MB, int P, int num_blocks,
                                                  int32_t *__restrict__ status)
{
    __shared__ int bad, first, kinds;
    if (threadIdx.x == 0) {
        bad = 0;
        first = 0x7FFFFFFF;
        kinds = 0;
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int b = wave; b < B; b += 16) {
        const long long L = seq_lens[b];
        int kind = (L < 0 || L > (long long)MB * P) ? 1 : 0;
        const int np = kind ? 0 : (int)((L + P - 1) / P);
        bool bad_block = false;
        for (int j = lane; j < np; j += 64) {
            const int id = block_table[(long long)b * MB + j];
            bad_block |= id < 0 || id >= num_blocks;
        }
        if (__any(bad_block))
            kind |= 2;
        if (kind && lane == 0) {
            atomicAdd(&bad, 1);
            atomicMin(&first, b);
            atomicOr(&kinds, kind);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        status[0] = bad;
        status[1] = bad ? first : -1;
        status[2] = kinds;
    }
}

// ===========================================================================
// host side
// ===========================================================================
bool valid_shape(const mla_decode_shape_t *s, mla_status_t *err)
{
    if (s->batch < 0 || s->num_heads <= 0 || s->num_blocks <= 0 || s->page_size <= 0 ||
        s->max_blocks_per_seq <= 0) {
        *err = MLA_ERR_BAD_SHAPE;
        return false;
    }
    if (s->kv_lora_rank != MLA_KV_LORA_RANK || s->qk_rope_head_dim != MLA_QK_ROPE_HEAD_DIM ||
        s->num_heads % 16 != 0) {
        *err = MLA_ERR_UNSUPPORTED;
        return false;
    }
    if (s->page_size < 16 || s->page_size > 1024 || (s->page_size & (s->page_size - 1))) {
        *err = MLA_ERR_UNSUPPORTED;
        return false;
    }
    if (s->cache_dtype != MLA_CACHE_BF16 && s->cache_dtype != MLA_CACHE_FP8_E4M3FN) {
        *err = MLA_ERR_UNSUPPORTED;
        return false;
    }
    // grid = B * S * head groups must fit a 1-D launch
    return true;
}

int log2_int(int v)
{
    int r = 0;
    while ((1 << r) < v)
        ++r;
    return r;
}

mla_status_t launch_split(const mla_decode_shape_t *s, const void *q, const void *cache,
                          const float *cache_scale, const int32_t *block_table,
                          const int32_t *seq_lens, float softmax_scale, int S,
                          float *part_out, float *part_lse, void *out, float *lse,
                          hipStream_t stream, int q_len = 1, int causal = 1)
{
    Params p;
    p.q = (const __bf16 *)q;
    p.cache = (const uint8_t *)cache;
    p.cache_scale = cache_scale;
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.part_out = part_out;
    p.part_lse = part_lse;
    p.out = (__bf16 *)out;
    p.lse = lse;
    p.scale_log2 = softmax_scale * kLog2e;
    p.B = s->batch;
    p.N = q_len * s->num_heads;     // heads of all query rows of a request
    p.NR = s->num_heads;
    p.S = S;
    p.MB = s->max_blocks_per_seq;
    p.num_blocks = s->num_blocks;
    p.page_shift = log2_int(s->page_size);
    p.QL = q_len;
    p.causal = causal;
    const bool direct = part_out == nullptr;
    const bool fp8 = s->cache_dtype == MLA_CACHE_FP8_E4M3FN;
    // Kernel choice by the heads of a request (all its query rows):
    //   a multiple of 64:  role-split kernel, 64 heads per workgroup
    //   otherwise:         16 heads per workgroup
    const int heads_per_wg = p.N % 64 == 0 ? 64 : 16;
    p.HG = p.N / heads_per_wg;
    const long long grid = (long long)s->batch * S * p.HG;
    if (grid > 0x7FFFFFFFLL)
        return MLA_ERR_UNSUPPORTED;
    const dim3 g((unsigned)grid);
    if (heads_per_wg == 64) {
        if (direct && fp8)
            hipLaunchKernelGGL((mla_split_ws<true, true>), g, dim3(512), 0, stream, p);
        else if (fp8)
            hipLaunchKernelGGL((mla_split_ws<false, true>), g, dim3(512), 0, stream, p);
        else if (direct)
            hipLaunchKernelGGL((mla_split_ws<true, false>), g, dim3(512), 0, stream, p);
        else
            hipLaunchKernelGGL((mla_split_ws<false, false>), g, dim3(512), 0, stream, p);
    } else if (fp8) {
        if (direct)
            hipLaunchKernelGGL((mla_split_h16<true, true>), g, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((mla_split_h16<false, true>), g, dim3(256), 0, stream, p);
    } else {
        if (direct)
            hipLaunchKernelGGL((mla_split_h16<true, false>), g, dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((mla_split_h16<false, false>), g, dim3(256), 0, stream, p);
    }
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t launch_merge(long long rows, int S, const float *part_out, const float *part_lse,
                          void *out, float *lse, hipStream_t stream)
{
    if (rows == 0)
        return MLA_OK;
    // Lanes own 8 columns (one wave per row) once there are enough rows to
    // fill the GPU, fewer columns (more waves per row) below that.  The
    // width changes only the launch, not the arithmetic of an element.
    const int cols = rows >= 2048 ? 8 : rows >= 512 ? 4 : rows >= 128 ? 2 : 1;
    const long long waves = rows * (kDV / (64 * cols));
    const long long blocks = (waves + 3) / 4;
    if (blocks > 0x7FFFFFFFLL)
        return MLA_ERR_UNSUPPORTED;
    const dim3 g((unsigned)blocks), blk(256);
    __bf16 *o = (__bf16 *)out;
    const int r = (int)rows;
    if (cols == 8)
        hipLaunchKernelGGL(mla_merge<8>, g, blk, 0, stream, part_out, part_lse, o, lse, r, S);
    else if (cols == 4)
        hipLaunchKernelGGL(mla_merge<4>, g, blk, 0, stream, part_out, part_lse, o, lse, r, S);
    else if (cols == 2)
        hipLaunchKernelGGL(mla_merge<2>, g, blk, 0, stream, part_out, part_lse, o, lse, r, S);
    else
        hipLaunchKernelGGL(mla_merge<1>, g, blk, 0, stream, part_out, part_lse, o, lse, r, S);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (mla_decode_noalloc): the split
// partials live in this file-scope device array instead of a caller
// workspace.  Each device that runs the library holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: its device address is fetched once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// passed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(160) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch array.
mla_status_t scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MLA_ERR_HIP;
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] {
        slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess && slot.ptr == nullptr)
            slot.err = hipErrorInvalidSymbol;
    });
    if (slot.err != hipSuccess)
        return MLA_ERR_HIP;
    *out = slot.ptr;
    return MLA_OK;
}

size_t partial_bytes(const mla_decode_shape_t *s, int S)
{
    return (size_t)s->batch * (size_t)s->num_heads * (size_t)S * (kDV + 1) * sizeof(float);
}

mla_status_t check_common(const mla_decode_shape_t *shape, const void *q, const void *cache,
                          const float *cache_scale, const int32_t *block_table,
                          const int32_t *seq_lens, int32_t S)
{
    if (!shape)
        return MLA_ERR_NULL_POINTER;
    mla_status_t err = MLA_OK;
    if (!valid_shape(shape, &err))
        return err;
    if (S < 1 || S > MLA_MAX_KV_SPLITS)
        return MLA_ERR_BAD_SPLITS;
    if (shape->batch > 0 && (!q || !cache || !block_table || !seq_lens))
        return MLA_ERR_NULL_POINTER;
    if (shape->cache_dtype == MLA_CACHE_FP8_E4M3FN ? cache_scale == nullptr
                                                    : cache_scale != nullptr)
        return cache_scale ? MLA_ERR_UNSUPPORTED : MLA_ERR_NULL_POINTER;
    return MLA_OK;
}

} // namespace

extern "C" {

const char *mla_status_string(mla_status_t status)
{
    switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL_POINTER: return "MLA_ERR_NULL_POINTER: a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "MLA_ERR_BAD_SHAPE: a dimension is negative or inconsistent";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape or dtype not handled by this build";
    case MLA_ERR_BAD_SPLITS: return "MLA_ERR_BAD_SPLITS: num_kv_splits outside [1, 256]";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: the HIP runtime rejected a launch";
    case MLA_ERR_SCRATCH_LIMIT:
        return "MLA_ERR_SCRATCH_LIMIT: the split partials of this call exceed the library's "
               "static scratch (MLA_NOALLOC_SCRATCH_BYTES = 160 MiB); call mla_decode with a "
               "workspace, or use fewer splits";
    }
    return "unknown mla_status_t";
}

size_t mla_decode_workspace_size(const mla_decode_shape_t *shape, int32_t num_kv_splits)
{
    if (!shape || num_kv_splits < 1 || num_kv_splits > MLA_MAX_KV_SPLITS || shape->batch < 0 ||
        shape->num_heads < 0)
        return 0;
    if (num_kv_splits == 1)
        return 0;
    return partial_bytes(shape, num_kv_splits);
}

mla_status_t mla_decode(const mla_decode_shape_t *shape, const void *q, const void *latent_cache,
                        const float *cache_scale, const int32_t *block_table,
                        const int32_t *seq_lens, float softmax_scale, int32_t num_kv_splits,
                        void *workspace, size_t workspace_bytes, void *out, float *lse,
                        hipStream_t stream)
{
    mla_status_t err = check_common(shape, q, latent_cache, cache_scale, block_table, seq_lens,
                                    num_kv_splits);
    if (err != MLA_OK)
        return err;
    if (shape->batch > 0 && !out)
        return MLA_ERR_NULL_POINTER;
    const size_t need = mla_decode_workspace_size(shape, num_kv_splits);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return MLA_ERR_WORKSPACE;
    if (shape->batch == 0)
        return MLA_OK;
    if (num_kv_splits == 1)
        return launch_split(shape, q, latent_cache, cache_scale, block_table, seq_lens,
                            softmax_scale, 1, nullptr, nullptr, out, lse, stream);
    float *part_out = (float *)workspace;
    float *part_lse = part_out + (size_t)shape->batch * shape->num_heads * num_kv_splits * kDV;
    err = launch_split(shape, q, latent_cache, cache_scale, block_table, seq_lens, softmax_scale,
                       num_kv_splits, part_out, part_lse, nullptr, nullptr, stream);
    if (err != MLA_OK)
        return err;
    return launch_merge((long long)shape->batch * shape->num_heads, num_kv_splits, part_out,
                        part_lse, out, lse, stream);
}

mla_status_t mla_decode_noalloc(const mla_decode_shape_t *shape, const void *q,
                                const void *latent_cache, const float *cache_scale,
                                const int32_t *block_table, const int32_t *seq_lens,
                                float softmax_scale, int32_t num_kv_splits, void *out, float *lse,
                                hipStream_t stream)
{
    mla_status_t err = check_common(shape, q, latent_cache, cache_scale, block_table, seq_lens,
                                    num_kv_splits);
    if (err != MLA_OK)
        return err;
    if (shape->batch > 0 && !out)
        return MLA_ERR_NULL_POINTER;
    const size_t need = mla_decode_workspace_size(shape, num_kv_splits);
    static_assert(kScratchBytes == MLA_NOALLOC_SCRATCH_BYTES, "documented scratch size");
    if (need > kScratchBytes)
        return MLA_ERR_SCRATCH_LIMIT;
    if (shape->batch == 0)
        return MLA_OK;
    void *ws = nullptr;
    if (need > 0) {
        err = scratch_address(&ws);
        if (err != MLA_OK)
            return err;
    }
    // the same kernels as mla_decode, with the scratch as its workspace
    return mla_decode(shape, q, latent_cache, cache_scale, block_table, seq_lens, softmax_scale,
                      num_kv_splits, ws, need, out, lse, stream);
}

mla_status_t mla_decode_partials(const mla_decode_shape_t *shape, const void *q,
                                 const void *latent_cache, const float *cache_scale,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 float softmax_scale, int32_t num_kv_splits, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream)
{
    mla_status_t err = check_common(shape, q, latent_cache, cache_scale, block_table, seq_lens,
                                    num_kv_splits);
    if (err != MLA_OK)
        return err;
    const size_t need = partial_bytes(shape, num_kv_splits);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return MLA_ERR_WORKSPACE;
    if (shape->batch == 0)
        return MLA_OK;
    float *part_out = (float *)workspace;
    float *part_lse = part_out + (size_t)shape->batch * shape->num_heads * num_kv_splits * kDV;
    return launch_split(shape, q, latent_cache, cache_scale, block_table, seq_lens, softmax_scale,
                        num_kv_splits, part_out, part_lse, nullptr, nullptr, stream);
}

size_t mla_decode_multi_workspace_size(const mla_decode_shape_t *shape, int32_t q_len,
                                       int32_t num_kv_splits)
{
    if (!shape || q_len < 1 || q_len > MLA_MAX_QUERY_LEN)
        return 0;
    mla_decode_shape_t v = *shape;
    v.batch = shape->batch * q_len;
    return mla_decode_workspace_size(&v, num_kv_splits);
}

mla_status_t mla_decode_multi(const mla_decode_shape_t *shape, int32_t q_len, int32_t causal,
                              const void *q, const void *latent_cache, const float *cache_scale,
                              const int32_t *block_table, const int32_t *seq_lens,
                              float softmax_scale, int32_t num_kv_splits, void *workspace,
                              size_t workspace_bytes, void *out, float *lse, hipStream_t stream)
{
    if (q_len < 1 || q_len > MLA_MAX_QUERY_LEN)
        return MLA_ERR_BAD_SHAPE;
    mla_status_t err = check_common(shape, q, latent_cache, cache_scale, block_table, seq_lens,
                                    num_kv_splits);
    if (err != MLA_OK)
        return err;
    if (shape->batch > 0 && !out)
        return MLA_ERR_NULL_POINTER;
    const size_t need = mla_decode_multi_workspace_size(shape, q_len, num_kv_splits);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return MLA_ERR_WORKSPACE;
    if (shape->batch == 0)
        return MLA_OK;
    const int c = causal ? 1 : 0;
    if (num_kv_splits == 1)
        return launch_split(shape, q, latent_cache, cache_scale, block_table, seq_lens,
                            softmax_scale, 1, nullptr, nullptr, out, lse, stream, q_len, c);
    const size_t rows = (size_t)shape->batch * q_len * shape->num_heads;
    float *part_out = (float *)workspace;
    float *part_lse = part_out + rows * num_kv_splits * kDV;
    err = launch_split(shape, q, latent_cache, cache_scale, block_table, seq_lens, softmax_scale,
                       num_kv_splits, part_out, part_lse, nullptr, nullptr, stream, q_len, c);
    if (err != MLA_OK)
        return err;
    return launch_merge((long long)rows, num_kv_splits, part_out, part_lse, out, lse, stream);
}

mla_status_t mla_merge_states(int32_t batch, int32_t num_heads, int32_t S, int32_t dv,
                              const float *part_out, const float *part_lse, void *out, float *lse,
                              hipStream_t stream)
{
    if (batch < 0 || num_heads < 0)
        return MLA_ERR_BAD_SHAPE;
    if (S < 1 || S > MLA_MAX_KV_SPLITS)
        return MLA_ERR_BAD_SPLITS;
    if (dv != kDV)
        return MLA_ERR_UNSUPPORTED;
    const long long rows = (long long)batch * num_heads;
    if (rows > 0x7FFFFFFFLL)
        return MLA_ERR_UNSUPPORTED;
    if (rows > 0 && (!part_out || !part_lse || !out))
        return MLA_ERR_NULL_POINTER;
    return launch_merge(rows, S, part_out, part_lse, out, lse, stream);
}

static mla_status_t launch_head_mm(int K, int M, int32_t batch, int32_t num_heads, const void *x,
                                   int64_t x_token_stride, int64_t x_head_stride, const void *w,
                                   void *out, hipStream_t stream)
{
    if (batch < 0 || num_heads < 0 || x_token_stride < 0 || x_head_stride < 0)
        return MLA_ERR_BAD_SHAPE;
    if (batch == 0 || num_heads == 0)
        return MLA_OK;
    if (!x || !w || !out)
        return MLA_ERR_NULL_POINTER;
    // 16-byte loads of x and of W rows
    if ((x_token_stride | x_head_stride) & 7 || ((uintptr_t)x & 15) || ((uintptr_t)w & 15) ||
        ((uintptr_t)out & 15))
        return MLA_ERR_UNSUPPORTED;
    // units of (head, column block, 64-row block): the absorb takes 128-column
    // blocks (32 KB of W each), the up-projection 64-column blocks (64 KB)
    const int mb = K == 128 ? 128 : 64;
    const long long grid = (long long)num_heads * (M / mb) * ((batch + 63) / 64);
    if (grid > 0x7FFFFFFFLL)
        return MLA_ERR_UNSUPPORTED;
    const dim3 g((unsigned)grid), blk(256);
    const __bf16 *xb = (const __bf16 *)x, *wb = (const __bf16 *)w;
    __bf16 *ob = (__bf16 *)out;
    const long long ts = x_token_stride, hs = x_head_stride;
    if (K == 128)
        hipLaunchKernelGGL((mla_head_mm<128, 128>), g, blk, 0, stream, xb, ts, hs, wb, ob, batch, num_heads, M);
    else
        hipLaunchKernelGGL((mla_head_mm<512, 64>), g, blk, 0, stream, xb, ts, hs, wb, ob, batch, num_heads, M);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_check_inputs(const mla_decode_shape_t *shape, const int32_t *block_table,
                              const int32_t *seq_lens, int32_t *status, hipStream_t stream)
{
    if (!shape || !status)
        return MLA_ERR_NULL_POINTER;
    mla_status_t err = MLA_OK;
    if (!valid_shape(shape, &err))
        return err;
    if (shape->batch > 0 && (!block_table || !seq_lens))
        return MLA_ERR_NULL_POINTER;
    hipLaunchKernelGGL(mla_check, dim3(1), dim3(1024), 0, stream, block_table, seq_lens,
                       shape->batch, shape->max_blocks_per_seq, shape->page_size,
                       shape->num_blocks, status);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_absorb_query(int32_t batch, int32_t num_heads, const void *q_nope,
                              int64_t q_token_stride, int64_t q_head_stride, const void *w_uk_t,
                              void *ql_nope, hipStream_t stream)
{
    return launch_head_mm(128, kDV, batch, num_heads, q_nope, q_token_stride, q_head_stride,
                          w_uk_t, ql_nope, stream);
}

mla_status_t mla_up_project(int32_t batch, int32_t num_heads, const void *latent_out,
                            int64_t x_token_stride, int64_t x_head_stride, const void *w_uv,
                            void *out, hipStream_t stream)
{
    return launch_head_mm(kDV, 128, batch, num_heads, latent_out, x_token_stride, x_head_stride,
                          w_uv, out, stream);
}

mla_status_t mla_gather_cache(int32_t num_tokens, const void *latent_cache, int32_t num_blocks,
                              int32_t page_size, mla_cache_dtype_t cache_dtype,
                              const float *cache_scale, const int32_t *block_table, int32_t batch,
                              int32_t max_blocks_per_seq, const int32_t *cu_seq_lens,
                              const int32_t *token_to_seq, const int32_t *seq_starts, void *dst,
                              hipStream_t stream)
{
    if (num_tokens < 0 || num_blocks < 0 || page_size < 1 || batch < 0 ||
        max_blocks_per_seq < 0)
        return MLA_ERR_BAD_SHAPE;
    if (cache_dtype != MLA_CACHE_BF16 && cache_dtype != MLA_CACHE_FP8_E4M3FN)
        return MLA_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype == MLA_CACHE_FP8_E4M3FN;
    if (num_tokens == 0)
        return MLA_OK;
    if (batch < 1 || max_blocks_per_seq < 1 || num_blocks < 1)
        return MLA_ERR_BAD_SHAPE;
    if (!latent_cache || !block_table || !cu_seq_lens || !token_to_seq || !dst ||
        (fp8 && !cache_scale))
        return MLA_ERR_NULL_POINTER;
    const long long n = (long long)num_tokens * 18;
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFLL)
        return MLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(mla_gather, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint8_t *)latent_cache, fp8 ? 1 : 0, cache_scale, block_table, batch,
                       max_blocks_per_seq, num_blocks, page_size, cu_seq_lens, token_to_seq,
                       seq_starts, (__bf16 *)dst, n);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_merge_attn_states(int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                   const void *prefix_out, const float *prefix_lse,
                                   const void *suffix_out, const float *suffix_lse, void *out,
                                   float *out_lse, hipStream_t stream)
{
    if (num_tokens < 0 || num_heads < 0 || head_dim < 0)
        return MLA_ERR_BAD_SHAPE;
    if (head_dim < 8 || head_dim > 2048 || (head_dim & (head_dim - 1)) != 0)
        return MLA_ERR_UNSUPPORTED;
    if (num_tokens == 0 || num_heads == 0)
        return MLA_OK;
    if (!prefix_out || !prefix_lse || !suffix_out || !suffix_lse || !out)
        return MLA_ERR_NULL_POINTER;
    const long long n = (long long)num_tokens * num_heads * (head_dim / 8);
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFLL)
        return MLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(mla_merge_two, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const __bf16 *)prefix_out, prefix_lse, (const __bf16 *)suffix_out,
                       suffix_lse, (__bf16 *)out, out_lse, num_tokens, num_heads, head_dim, n);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_concat_q_insert_cache(int32_t num_tokens, int32_t num_heads,
                                       const void *ql_nope, const void *q_pe, const void *kv_c,
                                       const void *k_pe, const int64_t *slot_mapping,
                                       int32_t num_blocks, int32_t page_size,
                                       mla_cache_dtype_t cache_dtype, const float *cache_scale_inv,
                                       void *latent_cache, void *q_out, hipStream_t stream)
{
    if (num_tokens < 0 || num_heads < 0 || num_blocks < 0 || page_size < 1)
        return MLA_ERR_BAD_SHAPE;
    if (cache_dtype != MLA_CACHE_BF16 && cache_dtype != MLA_CACHE_FP8_E4M3FN)
        return MLA_ERR_UNSUPPORTED;
    const bool fp8 = cache_dtype == MLA_CACHE_FP8_E4M3FN;
    if (num_tokens == 0)
        return MLA_OK;
    if (!kv_c || !k_pe || !slot_mapping || !latent_cache || (fp8 && !cache_scale_inv))
        return MLA_ERR_NULL_POINTER;
    if (num_heads > 0 && (!ql_nope || !q_pe || !q_out))
        return MLA_ERR_NULL_POINTER;
    const long long nq = (long long)num_tokens * num_heads * 72;
    const long long total = nq + (long long)num_tokens * (fp8 ? 36 : 72);
    const long long blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFFLL)
        return MLA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(mla_concat_insert, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const __bf16 *)ql_nope, (const __bf16 *)q_pe, (const __bf16 *)kv_c,
                       (const __bf16 *)k_pe, slot_mapping, (uint8_t *)latent_cache,
                       (__bf16 *)q_out, cache_scale_inv, nq, num_tokens,
                       (long long)num_blocks * page_size, fp8 ? 1 : 0);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

} // extern "C"
