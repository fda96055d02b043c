// MSA indexer: index scores of every cached key against the index queries, max-pooled into one
// score per 128-token block.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": one index query per GQA
// group scores every key of the single shared index-key head; scores are max-pooled per block;
// the scan reads only the index keys of the whole context each step (the term that still grows
// with context). "MiniMax M3 on vLLM", section "Decode indexer score kernel": a dedicated score
// kernel, not a padded dense GEMM, keeping the top-k boundary close to the scores; section "MSA
// mechanism": the partial last block and the causal boundary are masked.
//
// Work split: a workgroup of four wavefront pairs takes 32 consecutive blocks of one sequence;
// a pair takes 8 of them (a block never spans two pages, so the max-pool stays inside the pair),
// and wavefront h of the pair scores the 64 tokens of half h of each page. Pages stream into
// LDS with direct global->LDS loads, one half page ahead of the one being scored, so eight
// wavefronts per CU (two per SIMD) keep the loads in flight while the SIMDs dequantize: the
// dequantization, not the matrix cores, is most of the arithmetic, and a second wavefront per
// SIMD hides its latencies. The two half-page maxima of a block meet in LDS at the end.
// Per 16-token slab a wavefront dequantizes the keys exactly (A operand, tokens x dims) and
// multiplies them with up to 16 index-query rows (B operand, dims x rows; a row is (query
// token j, group g)) on the matrix cores, fp32 accumulate.
// Keys are dequantized to fp16 with one conversion and one packed multiply per pair of values
// (exact); the query rows are scaled by a power of two into fp16 range (exact for any row whose
// values span less than about 2^29) and the block maxima scaled back. A wavefront whose rows do
// not convert exactly takes the bf16 path (exact keys, bf16 queries) instead.
// Rows beyond 16 (q_len > 4) loop over row tiles.
#include "device_common.hpp"
#include "kernels.hpp"
#include "nvfp4_quant.hpp"

namespace msa {
namespace {

constexpr int kFusedMaxNew = 8;    // new tokens per sequence the fused step's patch stages
constexpr int kPairs = 4;            // wavefront pairs per workgroup; a pair shares its blocks
constexpr int kWaves = 2 * kPairs;   // wavefront h of a pair scores the tokens of half h of each page
constexpr int kBufs = 2;             // LDS buffers per wavefront (half pages in flight: kBufs - 1)
constexpr int kPagesPerWg = 32;     // blocks of one sequence per workgroup
static_assert(kPagesPerWg * 16 == kWaves * 64, "the score write-out: one thread per block and row");
constexpr int kHalfBytes = 5 * 1024; // four code slabs of a half page + the page's scale chunk

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kNonTemporal = 2;  // cache-policy bits of the DMA loads: stream, each page is read once

// Copy half h of a 9,216-byte page into this wavefront's LDS buffer with five direct
// global->LDS 16-byte loads, without registers: code slabs 4h..4h+3 (tokens with
// (t % 32) / 4 in that range) and the scale kilobyte (lane l's bytes land at buffer + 16 l of
// each kilobyte). Both wavefronts of a pair read the scale kilobyte, the second mostly from the
// L2: four-byte loads of each half's own scale words move the same bytes in more, smaller
// requests and measured slower.
__device__ __forceinline__ void half_to_lds(const uint8_t* pg, int h, uint8_t* buf, int lane) {
#pragma unroll
    for (int s = 0; s < 4; s++)
        __builtin_amdgcn_global_load_lds(pg + (4 * h + s) * 1024 + lane * 16,
                                         (lds_void*)(buf + s * 1024), 16, 0, kNonTemporal);
    __builtin_amdgcn_global_load_lds(pg + 8192 + lane * 16, (lds_void*)(buf + 4096), 16, 0,
                                     kNonTemporal);
}

// Wait until the loads of all but the `after` most recently issued half pages (five loads
// each) have completed. It is the compiler's own wait instruction (vmcnt only; expcnt 7 and
// lgkmcnt 15 wait for nothing), so the compiler knows which earlier loads have completed and
// adds no wait of its own for them later.
__device__ __forceinline__ void wait_halves(int after) {
    asm volatile("" ::: "memory");
    switch (after) {
        case 0: __builtin_amdgcn_s_waitcnt(0xF70); break;   // vmcnt(0)
        case 1: __builtin_amdgcn_s_waitcnt(0xF75); break;   // vmcnt(5)
        default: __builtin_amdgcn_s_waitcnt(0xF7A); break;  // vmcnt(10)
    }
    asm volatile("" ::: "memory");
}
static_assert(kBufs <= 3, "wait_halves covers at most two half pages in flight");

// This lane's query operand (four 16-byte pieces, piece m at q + 1024 m + 16 lane) read from
// LDS, where direct global->LDS loads put it: no register is written by a load the compiler
// does not see, so no copy of one can be taken before its wait.
__device__ __forceinline__ void read_query(u32x4 (&v)[4], const uint8_t* q, int lane) {
    const uint32_t a = (uint32_t)(uintptr_t)(q + lane * 16);
    asm volatile("ds_read_b128 %0, %4\n\t"
                 "ds_read_b128 %1, %4 offset:1024\n\t"
                 "ds_read_b128 %2, %4 offset:2048\n\t"
                 "ds_read_b128 %3, %4 offset:3072\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(a) : "memory");
}

// This lane's four 16-byte code chunks and the two scale words of its slabs, read from LDS
// with explicit instructions: the compiler would otherwise wait for every DMA load in flight
// before any LDS read, since it cannot tell which buffer the loads write.
struct HalfRegs {
    u32x4 code[4];
    uint32_t scale[2];
};
__device__ __forceinline__ void read_half(HalfRegs& hr, const uint8_t* buf, int h, int lane) {
    const uint32_t a = (uint32_t)(uintptr_t)(buf + lane * 16);
    const uint32_t as = (uint32_t)(uintptr_t)(buf + 4096 + lane * 16 + h * 8);
    // issued and waited for within one asm statement (no pending register outside it)
    asm volatile("ds_read_b128 %0, %6\n\t"
                 "ds_read_b128 %1, %6 offset:1024\n\t"
                 "ds_read_b128 %2, %6 offset:2048\n\t"
                 "ds_read_b128 %3, %6 offset:3072\n\t"
                 "ds_read_b32 %4, %7\n\t"
                 "ds_read_b32 %5, %7 offset:4\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(hr.code[0]), "=&v"(hr.code[1]), "=&v"(hr.code[2]), "=&v"(hr.code[3]),
                   "=&v"(hr.scale[0]), "=&v"(hr.scale[1])
                 : "v"(a), "v"(as)
                 : "memory");
}

// Max over this lane's 16 tokens of half h of a page (token 32c + 4s + i for slabs s = 4h..4h+3,
// query row n); masked -> -inf. `qop` holds the query operand as fp16 (F16 path) or as bf16
// bits (fallback); keys are dequantized to fp16 either way and, on the fallback, converted
// exactly to bf16.
template <bool FULL, bool F16>
__device__ __forceinline__ float half_max(const HalfRegs& hr, const u32x4 (&qop)[4], int h,
                                          int tok0, int c, int p_row) {
    float best = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < 4; s2++) {
        const int s = 4 * h + s2;
        f16x2 s0, s1;
        if (s2 & 1) e4m3_pair_f16<true>(hr.scale[s2 >> 1], s0, s1);
        else e4m3_pair_f16<false>(hr.scale[s2 >> 1], s0, s1);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const f16x8 a = dequant8_f16(hr.code[s2][m], m < 2 ? s0 : s1);
            if constexpr (F16)
                acc = mfma_f16_k32(a, __builtin_bit_cast(f16x8, qop[m]), acc);
            else
                acc = mfma_bf16_k32(f16x8_to_bf16x8(a), __builtin_bit_cast(bf16x8, qop[m]), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = tok0 + 32 * c + 4 * s + i;
            best = fmaxf(best, (FULL || t <= p_row) ? acc[i] : -INFINITY);
        }
    }
    return best;
}


// Fused decode step: the step's new tokens (positions T - q_len .. T - 1) are written to the
// caches by other wavefronts of the same launch, so a page of new tokens may still hold their
// old bytes when it streams in. The wavefront scoring half h of such a page writes the NVFP4
// bytes of those of the new index keys that fall in its half into its LDS copy of the page,
// exactly where the insert writes them in memory (the token's code chunks of the half and its
// scale bytes, which only this half reads). Such a page is always one of the two highest
// visible blocks of the row tile, the fixed first pages of wavefront pairs 0 and 1 (pages are
// scored from the highest block down), so only those wavefronts patch. One that does copies the
// sequence's new index keys (fp32) into its own staging area `pq` (token j at pq + 512 j; no
// workgroup barrier: only the wavefront itself reads them) with the query rows of the tile, and
// prepare_patch_token quantizes each token it needs once, overwriting the token's first 72 bytes
// with the result: the code byte of lane l's elements 2l, 2l+1 at pq + 512 j + l, scale g at
// pq + 512 j + 64 + g.
constexpr int kStageBytes = kDim * 4;

// Tokens j (bit j) of the step whose position lies in block blk and in half h of it.
__device__ __forceinline__ uint32_t patch_tokens(int blk, int T, int q_len, int h) {
    uint32_t mask = 0;
    for (int j = 0; j < q_len; j++) {
        const int pos = T - q_len + j;
        if (pos >= 0 && (pos >> 7) == blk && ((pos & 31) >> 4) == h) mask |= 1u << j;
    }
    return mask;
}

__device__ __forceinline__ void prepare_patch_token(uint8_t* pq, int j, int lane) {
    const uint32_t a = (uint32_t)(uintptr_t)(pq + kStageBytes * j);
    f32x2 x;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(a + 8 * lane)
                 : "memory");
    uint32_t byte, scale;
    quantize_pair(x[0], x[1], byte, scale);
    asm volatile("ds_write_b8 %0, %1" ::"v"(a + lane), "v"(byte) : "memory");
    if ((lane & 7) == 0)
        asm volatile("ds_write_b8 %0, %1" ::"v"(a + 64 + (lane >> 3)), "v"(scale) : "memory");
}

__device__ __forceinline__ void patch_new_tokens(const uint8_t* buf, int tok0, int T, int q_len,
                                                 int h, int lane, const uint8_t* pq) {
    const int first = max(T - q_len, tok0), last = min(T - 1, tok0 + kBlock - 1);
    for (int pos = first; pos <= last; pos++) {
        const int t = pos - tok0;
        if (((t & 31) >> 4) != h) continue;
        const uint32_t a = (uint32_t)(uintptr_t)(pq + kStageBytes * (pos - (T - q_len)));
        uint32_t byte, scale;
        asm volatile("ds_read_u8 %0, %2\n\tds_read_u8 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(byte), "=&v"(scale) : "v"(a + lane), "v"(a + 64 + (lane >> 3))
                     : "memory");
        const int sl = ((t & 31) >> 2) - 4 * h;  // the token's code slab within the half
        const uint32_t cb = (uint32_t)(uintptr_t)buf + sl * 1024 +
                            (16 * (lane >> 4) + 4 * (t >> 5) + (t & 3)) * 16 + (lane & 15);
        asm volatile("ds_write_b8 %0, %1" ::"v"(cb), "v"(byte) : "memory");
        if ((lane & 7) == 0) {
            const int g = lane >> 3;
            const uint32_t sb = (uint32_t)(uintptr_t)buf + 4096 + (g >> 1) * 256 + (t >> 5) * 64 +
                                (t & 3) * 16 + ((t & 31) >> 2) * 2 + (g & 1);
            asm volatile("ds_write_b8 %0, %1" ::"v"(sb), "v"(scale) : "memory");
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// A 64-bit value that is the same in every lane, as a scalar. (readfirstlane returns a signed
// int: each half goes through uint32_t so that the low half is not sign-extended.)
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (uint64_t)lo | ((uint64_t)hi << 32);
}

// A device-memory pointer rebuilt from its bits, marked global: left generic, its accesses
// would be flat instructions, which also count in the LDS counter and make the compiler wait
// for every load in flight before each of them.
template <typename T>
__device__ __forceinline__ T* global_ptr(uint64_t v) {
    typedef __attribute__((address_space(1))) T global_t;
    return (T*)(global_t*)v;
}

// Source of insert item i = 9 j + vec of sequence b: new token j, head vector vec (K heads
// 0-3, V heads 4-7, the index key 8).
__device__ __forceinline__ const float* item_source(int item, int b, int q_len,
                                                    const float* new_k, const float* new_v,
                                                    const float* new_ik) {
    const int j = item / 9, vec = item - 9 * (item / 9);
    const int64_t token = (int64_t)b * q_len + j;
    return vec < 4   ? new_k + (token * kKvHeads + vec) * kDim
           : vec < 8 ? new_v + (token * kKvHeads + vec - 4) * kDim
                     : new_ik + token * kDim;
}

// Store insert item i of sequence b (quantized to byte / scale by this wavefront) at position
// T - q_len + j, on page `page` (the block-table entry of that position).
__device__ __forceinline__ void store_item(int item, int64_t page, int pos, int64_t num_pages,
                                           uint32_t byte, uint32_t scale, uint8_t* k_pool,
                                           uint8_t* v_pool, uint8_t* ik_pool, int lane) {
    if (pos < 0 || page < 0 || page >= num_pages) return;
    const int vec = item - 9 * (item / 9);
    uint8_t* dst = vec < 4   ? k_pool + (page * kKvHeads + vec) * kHeadPageBytes
                   : vec < 8 ? v_pool + (page * kKvHeads + vec - 4) * kHeadPageBytes
                             : ik_pool + page * kHeadPageBytes;
    store_quantized(byte, scale, dst, pos & 127, vec >= 4 && vec < 8, lane);
}

// Claim the next unscored page of this half for the wavefront: one lane adds to the counter.
__device__ __forceinline__ int claim_page(const int* counter, int lane) {
    int old = 0;
    if (lane == 0)
        asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(old) : "v"((uint32_t)(uintptr_t)counter), "v"(1) : "memory");
    return __builtin_amdgcn_readfirstlane(old);
}

// One workgroup scores blocks [kPagesPerWg x, kPagesPerWg (x + 1)) of sequence b for every query
// row, one row tile (16 rows: four query tokens x four groups) at a time. Wavefront w = 2 m + h
// scores half h of a page (tokens with (t % 32) / 16 == h); the two halves of a page meet in the
// LDS stash. Pages are handed out dynamically, from the highest visible block down: wavefront
// pair m starts with page m, then each wavefront claims the next page of its half from an LDS
// counter, so that the wavefronts that run ahead (the older wavefront of each SIMD gets the
// issue slots first) take more pages and the workgroup finishes together. The half page of the
// next claimed page streams into LDS while the current one is scored.
//
// FUSED (decode step with q_len <= kFusedMaxNew): the launch also inserts the step's new tokens.
// The 9 q_len head vectors of sequence b are spread over the sequence's workgroups and their
// wavefronts (wavefront w of workgroup x takes items x + gx (w + 8 m)). A wavefront loads its
// first item with its start-up loads, requests the item's block-table entry after its first
// page, quantizes while the first pages stream in, and stores after its last page has arrived,
// so that the stores never stand between page loads in the in-order memory counter (stores
// issued after the first page measured 1.1 us slower). The barrier that follows waits for the
// LDS writes only, not for these stores. The
// indexer wavefronts patch the new index keys into their page copies (patch_new_tokens): a
// page may be read before or after another workgroup's store lands.
//
// A shard of the blocks (not FUSED): the table's column c holds the page of global block
// g_begin + c * g_stride, whose tokens sit at positions 128 (g_begin + c g_stride) onwards, and
// the context is clamped to total_blocks blocks (the whole table's width); column c of the
// scores is then the full indexer's column g_begin + c g_stride, bit for bit (every block's score
// is computed on its own, in the same order of operations).
template <bool FUSED>
__global__ __launch_bounds__(kWaves * 64) void indexer_kernel(
    const uint8_t* ik_pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_lens, int max_blocks, int q_len,
    const uint16_t* __restrict__ q_idx, float* __restrict__ scores, uint8_t* k_pool_w,
    uint8_t* v_pool_w, const float* __restrict__ new_k,
    const float* __restrict__ new_v, const float* __restrict__ new_ik, int g_begin, int g_stride,
    int total_blocks) {
    // the fused step scores the whole table
    const int gb = FUSED ? 0 : g_begin;
    const int gs = FUSED ? 1 : g_stride;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves][kBufs][kHalfBytes];
    // half-page maxima of the row tile: [half][row][block - wg_blk0], rows padded apart in banks
    __shared__ float stash[2][16][kPagesPerWg + 1];
    __shared__ int next_page[2];  // page counters of the two halves
    __shared__ __attribute__((aligned(8))) uint64_t fused_ptrs[FUSED ? kWaves : 1][5];
    __shared__ __attribute__((aligned(16))) uint8_t qbuf[kWaves][4 * 1024];  // query operands
    __shared__ __attribute__((aligned(16))) uint8_t stage[FUSED ? 4 : 1][FUSED ? kFusedMaxNew * kStageBytes : 16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gx = (max_blocks + kPagesPerWg - 1) / kPagesPerWg;
    const int wg = blockIdx.x;
    const int b = wg / gx;
    const int wg_blk0 = (wg - b * gx) * kPagesPerWg;
    const int wg_end = min(wg_blk0 + kPagesPerWg, max_blocks);
    const int n_items = FUSED ? 9 * q_len : 0;
    int item = (wg - b * gx) + gx * __builtin_amdgcn_readfirstlane(wave);  // first insert item
    const int pair = __builtin_amdgcn_readfirstlane(wave >> 1);
    const int h = wave & 1;
    const int n = lane & 15;  // B/D column: query row within the tile
    const int c = lane >> 4;  // lane group
    const int32_t* table = block_table + (int64_t)b * max_blocks;
    // the page counters are set before any wavefront claims a page (and before the start-up
    // loads, so that the barrier does not wait for them)
    if (threadIdx.x < 2) {
        const uint32_t a = (uint32_t)(uintptr_t)&next_page[threadIdx.x];
        asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(kPairs) : "memory");
    }
    __builtin_amdgcn_s_barrier();
    // the workgroup's block-table entries (lane l: block wg_blk0 + l) and the context length are
    // requested together (the entries do not depend on it): one memory round trip before the
    // first page load; and, fused, this wavefront's first insert item
    int pid_all = -1;
    if (wg_blk0 + lane < wg_end && lane < kPagesPerWg) pid_all = table[wg_blk0 + lane];
    int T_raw = ctx_lens[b];
    f32x2 ins_x = {0.f, 0.f};
    if constexpr (FUSED) {
        if (item < n_items)
            ins_x = *reinterpret_cast<const f32x2*>(
                item_source(item, b, q_len, new_k, new_v, new_ik) + 2 * lane);
        // pairs 0 and 1 (the wavefronts whose first pages may hold new tokens): the sequence's
        // new index keys into their staging area, two tokens per direct global->LDS load
        // (lanes past the last token re-read its last 16 bytes into the unused tail), with the
        // start-up loads, so that the first page request waits for nothing of the patch
        if (pair < 2) {
            const float* src = new_ik + (int64_t)b * q_len * kDim;
            for (int i = 0; i < (q_len + 1) / 2; i++)
                __builtin_amdgcn_global_load_lds(src + min(256 * i + 4 * lane, q_len * kDim - 4),
                                                 (lds_void*)(stage[pair * 2 + h] + 1024 * i), 16,
                                                 0, 0);
        }
    }
    asm volatile("" : "+v"(pid_all), "+v"(T_raw), "+v"(ins_x));
    // the same value in every lane
    const int T = __builtin_amdgcn_readfirstlane(clamp_ctx(T_raw, FUSED ? max_blocks : total_blocks));
    MSA_CHECK(threadIdx.x != 0 || (T_raw >= q_len && T_raw <= (FUSED ? max_blocks : total_blocks) * kBlock),
              kCheckCtxLen);
    const int rows = 4 * q_len;
    const int64_t row_base = (int64_t)b * rows;
    // blocks past the last query position hold no visible key and are never loaded (columns
    // below n_blocks hold a global block below the context's block count)
    const int nb_ctx = T > 0 ? (T - 1) / kBlock + 1 : 0;
    const int n_blocks = nb_ctx > gb ? min(max_blocks, (nb_ctx - gb + gs - 1) / gs) : 0;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    pid_all = (wg_blk0 + lane < n_blocks && pid_all >= 0 && pid_all < num_pages) ? pid_all : -1;
    if (wg_blk0 >= n_blocks) {
        // no block of this workgroup holds a key of the context (a short sequence in a batch
        // sized for a longer one): every score of its blocks is -inf, and the workgroup ends
        // after its insert items, freeing its compute unit a memory round trip sooner
        const int rows_all = 4 * q_len;
        for (int i = threadIdx.x; i < rows_all * kPagesPerWg; i += kWaves * 64) {
            const int rn = i / kPagesPerWg, kb = i - rn * kPagesPerWg;
            if (wg_blk0 + kb < wg_end)
                scores[((int64_t)b * rows_all + rn) * max_blocks + wg_blk0 + kb] = -INFINITY;
        }
        if constexpr (FUSED) {
            for (bool first = true; item < n_items; item += kWaves * gx, first = false) {
                const f32x2 x = first ? ins_x
                                      : *reinterpret_cast<const f32x2*>(
                                            item_source(item, b, q_len, new_k, new_v, new_ik) + 2 * lane);
                const int pos = T - q_len + item / 9;
                const int64_t page = pos >= 0 ? table[pos >> 7] : -1;
                uint32_t byte, scale;
                quantize_pair(x[0], x[1], byte, scale);
                store_item(item, page, pos, num_pages, byte, scale, k_pool_w, v_pool_w,
                           const_cast<uint8_t*>(ik_pool), lane);
            }
        }
        return;
    }
    // the first insert item's position and block-table entry (set after the first page of the
    // first row tile is requested)
    int ins_pos = -1;
    int ins_page_v = -1;
    uint32_t ins_byte = 0, ins_scale = 0;
    uint32_t prepped = 0;  // fused: tokens whose patch bytes are in this wavefront's staging area

    // row tile rt (query rows rt .. rt + 15): one past its highest visible column; page u of
    // the tile is column vis_end - 1 - u
    auto tile_vis_end = [&](int rt) {
        const int p_hi = T - q_len + min((rt >> 2) + 3, q_len - 1);  // highest position in it
        const int hb = p_hi >= 0 ? p_hi / kBlock : -1;                // its global block
        return min(wg_end, hb >= gb ? (hb - gb) / gs + 1 : 0);
    };
    // load half h of page u of a tile into LDS buffer `buf`; false when the page is absent
    auto issue = [&](int u, int buf, int vis_end) {
        MSA_CHECK(vis_end - 1 - u - wg_blk0 >= 0 && vis_end - 1 - u - wg_blk0 < kPagesPerWg, kCheckLds);
        const int pid = __builtin_amdgcn_readlane(pid_all, vis_end - 1 - u - wg_blk0);
        if (pid < 0) return false;
        half_to_lds(ik_pool + (int64_t)pid * kHeadPageBytes, h, lds[wave][buf], lane);
        return true;
    };
    // request a row tile's loads: the patch staging (fused, pairs 0 and 1), the query rows and
    // this wavefront's first page
    auto request_tile = [&](int rt, uint32_t& patch_mask, int& cur, bool& cur_loaded) {
        const int vis_end = tile_vis_end(rt);
        const int n_pages = max(vis_end - wg_blk0, 0);
        // fused: the tokens this wavefront patches into its first page (pairs 0 and 1 only)
        patch_mask = 0;
        if constexpr (FUSED) {
            if (pair < 2 && pair < n_pages)
                patch_mask = patch_tokens(vis_end - 1 - pair, T, q_len, h);
        }
        // B operand: row r, dims 32c + 8m .. 32c + 8m + 7 for MFMA m = 0..3, copied into this
        // wavefront's query buffer with direct global->LDS loads, requested before the first
        // page: the wait for it leaves the page in flight. Every lane loads a valid row (rows
        // past the tile read row rows - 1) and zeroes it after the wait.
        {
            const uint16_t* qp = q_idx + (row_base + min(rt + n, rows - 1)) * kDim + 32 * c;
#pragma unroll
            for (int m = 0; m < 4; m++)
                __builtin_amdgcn_global_load_lds(qp + 8 * m, (lds_void*)(qbuf[wave] + 1024 * m),
                                                 16, 0, 0);
        }
        cur = pair < n_pages ? pair : n_pages;  // this wavefront's page (n_pages: none)
        cur_loaded = cur < n_pages && issue(cur, 0, vis_end);
    };
    // fused: the insert's source and destination pointers, kept in LDS (not live in scalar
    // registers through the scan)
    auto insert_ptrs = [&](uint64_t (&fp)[5]) {
        const uint32_t a = (uint32_t)(uintptr_t)&fused_ptrs[wave][0];
        asm volatile("ds_read_b64 %0, %5\n\tds_read_b64 %1, %5 offset:8\n\t"
                     "ds_read_b64 %2, %5 offset:16\n\tds_read_b64 %3, %5 offset:24\n\t"
                     "ds_read_b64 %4, %5 offset:32\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(fp[0]), "=&v"(fp[1]), "=&v"(fp[2]), "=&v"(fp[3]), "=&v"(fp[4])
                     : "v"(a) : "memory");
    };
    uint32_t patch_mask;
    int cur;
    bool cur_loaded;
    // the first tile's loads go out right after start-up, ahead of any other set-up
    request_tile(0, patch_mask, cur, cur_loaded);

    for (int rt = 0; rt < rows; rt += 16) {
        const int r = rt + n;
        const int p_row = T - q_len + (r >> 2);                  // position of row r's token
        const int p_lo = T - q_len + (rt >> 2);                  // lowest position in the tile
        const int vis_end = tile_vis_end(rt);
        const int n_pages = max(vis_end - wg_blk0, 0);
        if (rt > 0) request_tile(rt, patch_mask, cur, cur_loaded);
        if constexpr (FUSED) {
            if (rt == 0 && item < n_items) {
                // after the first loads are issued (the item's work never delays them): the
                // item's block-table entry, a load the compiler sees (vector, through an index it
                // cannot prove uniform) and waits for at its use, the store after the last page;
                // and its quantization, while the first page is in flight
                int t_late = T;
                asm volatile("" : "+v"(t_late));
                ins_pos = __builtin_amdgcn_readfirstlane(t_late) - q_len + item / 9;
                if (ins_pos >= 0) {
                    int idx = ins_pos >> 7;
                    asm volatile("" : "+v"(idx));
                    ins_page_v = table[idx];
                }
                quantize_pair(ins_x[0], ins_x[1], ins_byte, ins_scale);
                // the insert's pointers, needed again only by the stores after the last page,
                // kept in this wavefront's LDS slot rather than in scalar registers through the
                // scan (written here, off the start-up path, and read back by this wavefront)
                if (lane == 0) {
                    const uint32_t a = (uint32_t)(uintptr_t)&fused_ptrs[wave][0];
                    const uint64_t p0 = (uint64_t)(uintptr_t)new_k, p1 = (uint64_t)(uintptr_t)new_v;
                    const uint64_t p2 = (uint64_t)(uintptr_t)new_ik, p3 = (uint64_t)(uintptr_t)k_pool_w;
                    const uint64_t p4 = (uint64_t)(uintptr_t)v_pool_w;
                    asm volatile("ds_write_b64 %0, %1\n\tds_write_b64 %0, %2 offset:8\n\t"
                                 "ds_write_b64 %0, %3 offset:16\n\tds_write_b64 %0, %4 offset:24\n\t"
                                 "ds_write_b64 %0, %5 offset:32\n\ts_waitcnt lgkmcnt(0)"
                                 ::"v"(a), "v"(p0), "v"(p1), "v"(p2), "v"(p3), "v"(p4) : "memory");
                }
            }
        }
        wait_halves(cur_loaded ? 1 : 0);
        u32x4 qraw[4];
        read_query(qraw, qbuf[wave], lane);
        bf16x8 qb[4];
#pragma unroll
        for (int m = 0; m < 4; m++)
            qb[m] = r < rows ? __builtin_bit_cast(bf16x8, qraw[m]) : bf16x8{};
        f16x8 qh[4];
        float out_scale;
        const bool f16 = __all(query_to_f16(qb, qh, out_scale));
        u32x4 qop[4];
#pragma unroll
        for (int m = 0; m < 4; m++)
            qop[m] = f16 ? __builtin_bit_cast(u32x4, qh[m]) : __builtin_bit_cast(u32x4, qb[m]);
        if (!f16) out_scale = 1.0f;
        if constexpr (FUSED) {
            // patch bytes of the tokens of the first page (staged at start-up)
            for (uint32_t todo = patch_mask & ~prepped; todo; todo &= todo - 1) {
                prepare_patch_token(stage[pair * 2 + h], __builtin_ctz(todo), lane);
            }
            prepped |= patch_mask;
        }

        int buf = 0;
#pragma unroll 1
        while (cur < n_pages) {
            const int nxt = claim_page(&next_page[h], lane);
            const bool nxt_loaded = nxt < n_pages && issue(nxt, buf ^ 1, vis_end);
            const int blk = vis_end - 1 - cur;
            const int tok0 = (gb + blk * gs) * kBlock;
            float best = -INFINITY;
            if (cur_loaded) {
                wait_halves(nxt_loaded ? 1 : 0);
                if constexpr (FUSED) {
                    if (cur == pair && patch_mask)
                        patch_new_tokens(lds[wave][buf], tok0, T, q_len, h, lane,
                                         stage[pair * 2 + h]);
                }
                HalfRegs hr;
                read_half(hr, lds[wave][buf], h, lane);
                const bool full = tok0 + kBlock - 1 <= p_lo;
                if (f16)
                    best = (full ? half_max<true, true>(hr, qop, h, tok0, c, p_row)
                                 : half_max<false, true>(hr, qop, h, tok0, c, p_row)) * out_scale;
                else
                    best = full ? half_max<true, false>(hr, qop, h, tok0, c, p_row)
                                : half_max<false, false>(hr, qop, h, tok0, c, p_row);
            }
            best = max_over_c(best);
            // kept in LDS until the tile ends: a global store here would join the page loads in
            // the in-order memory counter and make the next wait cover part of a later page
            if (c == 0) {
                const uint32_t a = (uint32_t)(uintptr_t)&stash[h][n][blk - wg_blk0];
                asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(best) : "memory");
            }
            cur = nxt;
            cur_loaded = nxt_loaded;
            buf ^= 1;
        }
        if constexpr (FUSED) {
            // the insert stores, after the wavefront's last page load has returned; then any
            // further items (more items than wavefronts: short contexts), one at a time
            if (rt + 16 >= rows && item < n_items) {
                uint64_t fp[5];
                insert_ptrs(fp);
                const float* nk = global_ptr<const float>(uniform64(fp[0]));
                const float* nv = global_ptr<const float>(uniform64(fp[1]));
                const float* nik = global_ptr<const float>(uniform64(fp[2]));
                uint8_t* kp = global_ptr<uint8_t>(uniform64(fp[3]));
                uint8_t* vpw = global_ptr<uint8_t>(uniform64(fp[4]));
                store_item(item, __builtin_amdgcn_readfirstlane(ins_page_v), ins_pos, num_pages,
                           ins_byte, ins_scale, kp, vpw, const_cast<uint8_t*>(ik_pool), lane);
                for (item += kWaves * gx; item < n_items; item += kWaves * gx) {
                    const f32x2 x = *reinterpret_cast<const f32x2*>(
                        item_source(item, b, q_len, nk, nv, nik) + 2 * lane);
                    const int pos = T - q_len + item / 9;
                    const int64_t page = pos >= 0 ? table[pos >> 7] : -1;
                    quantize_pair(x[0], x[1], ins_byte, ins_scale);
                    store_item(item, page, pos, num_pages, ins_byte, ins_scale, kp, vpw,
                               const_cast<uint8_t*>(ik_pool), lane);
                }
            }
        }
        // every page and query load has been waited for; the insert stores may still be in
        // flight and are left to complete on their own
        if constexpr (FUSED)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        // a plain barrier: the stash is in LDS, waited for above (a barrier with a fence would
        // also wait for the insert stores)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // thread (row rn, block slot kb) writes the max of both halves; blocks above the tile's
        // visible range are -inf; the counters are reset for the next tile
        {
            const int rn = threadIdx.x >> 5, kb = threadIdx.x & 31;
            if (wg_blk0 + kb < wg_end && rt + rn < rows)
                scores[(row_base + rt + rn) * max_blocks + wg_blk0 + kb] =
                    wg_blk0 + kb < vis_end ? fmaxf(stash[0][rn][kb], stash[1][rn][kb])
                                           : -INFINITY;
            if (threadIdx.x < 2) next_page[threadIdx.x] = kPairs;
        }
        __syncthreads();  // the next row tile rewrites the stash and claims pages anew
    }
}

}  // namespace

#ifdef MSA_CHECKED
MSA_DEFINE_CHECKS_READER(checks_take_indexer)
#endif

static int indexer_wgs(int batch, int max_blocks) {
    return (max_blocks + kPagesPerWg - 1) / kPagesPerWg * batch;
}

hipError_t launch_indexer_shard(const uint8_t* ik_pool, int64_t num_pages,
                                const int32_t* block_table, const int32_t* ctx_lens, int batch,
                                int max_blocks, int q_len, const uint16_t* q_idx, float* scores,
                                int block_begin, int block_stride, int total_blocks,
                                hipStream_t stream) {
    if (q_len >= kIndexerGemmMinQ)
        return launch_indexer_gemm_shard(ik_pool, num_pages, block_table, ctx_lens, batch,
                                         max_blocks, q_len, q_idx, scores, block_begin,
                                         block_stride, total_blocks, stream);
    hipLaunchKernelGGL(indexer_kernel<false>, dim3(indexer_wgs(batch, max_blocks)),
                       dim3(kWaves * 64), 0, stream, ik_pool, num_pages, block_table, ctx_lens,
                       max_blocks, q_len, q_idx, scores, nullptr, nullptr, nullptr, nullptr,
                       nullptr, block_begin, block_stride, total_blocks);
    return hipGetLastError();
}

hipError_t launch_indexer(const uint8_t* ik_pool, int64_t num_pages, const int32_t* block_table,
                          const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                          const uint16_t* q_idx, float* scores, hipStream_t stream) {
    return launch_indexer_shard(ik_pool, num_pages, block_table, ctx_lens, batch, max_blocks,
                                q_len, q_idx, scores, 0, 1, max_blocks, stream);
}

hipError_t launch_insert_indexer(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool,
                                 int64_t num_pages, const int32_t* block_table,
                                 const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                                 const float* new_k, const float* new_v, const float* new_ik,
                                 const uint16_t* q_idx, float* scores, hipStream_t stream) {
    if (q_len <= kFusedMaxNew) {
        hipLaunchKernelGGL(indexer_kernel<true>, dim3(indexer_wgs(batch, max_blocks)),
                           dim3(kWaves * 64), 0, stream, ik_pool, num_pages, block_table, ctx_lens,
                           max_blocks, q_len, q_idx, scores, k_pool, v_pool, new_k, new_v, new_ik,
                           0, 1, max_blocks);
        return hipGetLastError();
    }
    // more new tokens than the patch stages: the insert launch first, then the indexer
    const hipError_t err =
        launch_insert_at_positions(k_pool, v_pool, ik_pool, num_pages, block_table, ctx_lens,
                                   batch, max_blocks, q_len, new_k, new_v, new_ik, stream);
    if (err != hipSuccess) return err;
    return launch_indexer(ik_pool, num_pages, block_table, ctx_lens, batch, max_blocks, q_len,
                          q_idx, scores, stream);
}

}  // namespace msa
