// Internal launch interface between the C ABI layer (lola_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lola {

constexpr int kMaxLambda = 1024;     // largest cache the kernels support
constexpr int kMaxChunk = 128;       // largest prefill chunk

// Per-(sequence, head) scratch used by one prefill call.  Offsets are in bytes from the start of the
// (b, h) block; every region starts on a 256-byte boundary.
struct WsLayout {
    int64_t per_bh;        // bytes per (b, h)
    int64_t phi_store;     // [n + lam + eta][D] T : phi(k) of every token the call scores, by source index,
                           //   then [n][D] T: phi(q) of the call's queries (query-accumulated rules only)
    int64_t slot_pos;      // [lam] int32      : final cache table after the call (position, -1 empty)
    int64_t slot_src;      // [lam] int32      : where each final member's K/V come from (see Src below)
    int64_t mir_phi;       // [lam16/16][D/32][64][8] T: features of the cache slots, MFMA operand order
    int64_t mir_v;         // [lam16/16][d_v/32][64][2][4] T (bf16; fp32: [d_v/16][64][4]): cache slots' values, accumulator order
    int64_t chunk0;        // first per-chunk record
    int64_t per_chunk;     // bytes per chunk record
    // offsets inside a chunk record
    int64_t c_snap_h;      // [d_v/16][D/32][64][8] T: H at the chunk start, in MFMA fragment order
    int64_t c_snap_s;      // [D] fp32        : s at the chunk start
    int64_t c_cache_pos;   // [lam] int32     : cache after this chunk's allocation (positions)
    int64_t c_cache_src;   // [lam] int32     : their sources
    int64_t c_fold_n;      // int32           : number of tokens folded by this chunk
    int64_t c_fold_pos;    // [c_pad16] int32 : their positions
    int64_t c_fold_src;    // [c_pad16] int32 : their sources (features live in phi_store[src])
    int64_t c_fold_vt;     // [d_v][c_pad64] T: their values, transposed
    int32_t c_pad16;
    int32_t c_pad64;
    int32_t nchunks;
    int64_t score_alloc;   // [n + lam + eta] fp32: query-accumulated score a candidate has at its allocation
    int64_t score_full;    // [n + lam + eta] fp32: the same score with every query of the call
};

// A source index names where a token's K/V live during a prefill call:
//   0 <= src < n              : input row src of the call
//   n <= src < n + lam        : initial cache slot (src - n) of the state
//   n + lam <= src            : initial window ring slot (src - n - lam) of the state
// The commit kernel runs last, so the state's initial window and cache stay readable until then.

// Read-branch mask bits (which memories a query reads in Eq. (14)).
constexpr int kReadState = 1, kReadSparse = 2, kReadWindow = 4, kReadAll = 7;

// Cache-scoring rules: SRE, or a score accumulated over the queries whose window holds the key.
constexpr int kScoreSre = 0, kScoreKernelSq = 1, kScoreKernelAbs = 2, kScoreRatio = 3, kScoreAttn = 4;

struct PrefillArgs {
    int BH, n, C, eta, lam, nchunks, nqt;
    int c_begin, c_end;   // chunk range of one chain / read-out launch
    int64_t t0;
    const void* q;
    const void* k;
    const void* v;
    void* y;
    const float* W;
    float* H;             // [BH][d_v][D]
    float* s;             // [BH][D]
    void* win_k;
    void* win_v;
    void* cache_k;
    void* cache_v;
    int32_t* cache_pos;
    int32_t* fold_at;     // nullable
    char* ws;
    WsLayout L;
    // options (kept after the fields above: the chain kernel's code is sensitive to their layout)
    int read_mask;        // kRead* bits; always holds kReadWindow
    int score_rule;       // kScore*
    float* win_score;     // query-accumulated rules: the state's ring and cache scores
    float* cache_score;
};

struct DecodeArgs {
    int BH, eta, lam;
    int read_mask;        // kRead* bits; always holds kReadWindow
    int64_t t;
    const void* q;
    const void* k;
    const void* v;
    void* y;
    const float* W;
    float* H;
    float* s;
    void* win_k;
    void* win_v;
    void* cache_k;
    void* cache_v;
    int32_t* cache_pos;
    int32_t* folded_pos;  // nullable
    // chunked decode (dec_chunk > 1): the group's fold mask per (sequence, head), and whether this step
    // opens a group (allocation for the group's leaving tokens)
    int dec_chunk;
    int group_start;
    unsigned long long* dec_fold;
};

// SRE collision map of one prefill call, read from that call's workspace and the state it left.
struct CollideArgs {
    int BH, n, C, eta, nchunks;
    int nblk, tok_per_block;   // token blocks per map row and tokens per block
    int relative;
    const void* v;             // the call's values [BH][n][d_v]
    const int32_t* fold_at;    // the call's fold chunks [BH][n]
    const float* H;            // state after the call (the last row)
    const float* s;
    const char* ws;            // the call's workspace
    WsLayout L;                // its layout (same n and C)
    float* out;                // [BH][nchunks][n]
};
constexpr int kCollideTokensPerBlock = 256;
constexpr int kCollideRows = 2;           // map rows per workgroup (their H^T side by side in LDS)

// HOLA variant: a gated delta-rule state plus an exact cache chosen by write magnitude.
constexpr int kHolaMaxW = 64;     // largest persistent cache
constexpr int kHolaMaxC = 1024;   // largest chunk
struct HolaLayout {               // byte offsets of whole arrays in the workspace
    int64_t qinv, kinv;           // [BH][n] fp32: 1 / ||x||_2 of queries and keys (0 for a zero row)
    int64_t qtil, ktil;           // [BH][n][d] T   : RMS-normalised, gamma-scaled queries and keys
    int64_t o;                    // [BH][n][d] fp32: state read-out S_t^T q_t
    int64_t esq;                  // [BH][n][d / 16] fp32: sum of e_t^2 over each group of 16 value columns
    int64_t clist;                // [BH][nchunks + 1][kHolaMaxW] int32: persistent cache at each chunk start,
                                  // then after the last chunk (rank order)
    int64_t blk;                  // [BH][ceil(n / 16)] HolaBlock: the delta rule's per-block matrices
    int64_t sink;                 // [2][64] fp32: where the scan's stores for tokens past n go
    int64_t tlist;                // [BH][nchunks][min(kHolaMaxW, C)] u64: each chunk's own top-w ranking
                                  //   keys, largest first
    int64_t total;
};
// The delta rule over a block of 16 tokens (state S before the block, gates alpha, beta, unit keys and
// queries K, Q, values V):  E = T (V - diag(gam) K S),  O = diag(gam) Q S + M E,
// S' = glast S + K^T diag(wgt) E,  with gam_i = prod_{l <= i} alpha_l, T = (I + A)^{-1},
// A_ij = (prod_{j < l <= i} alpha_l) beta_j k_i.k_j (j < i), M_ij = (prod_{j < l <= i} alpha_l) beta_j q_i.k_j
// (j <= i), wgt_j = (prod_{l > j} alpha_l) beta_j, glast = gam_15.  T and M are stored as the A operand
// of a 16x16x4 MFMA: lane (g, r) holds row r, columns 4g .. 4g + 3.
constexpr int kHolaBT = 16;
struct HolaBlock {
    float Tp[64][4];
    float Mp[64][4];
    float gam[16];
    float wgt[16];
    float glast;
    float pad[3];
};
struct HolaArgs {
    int BH, heads, n, C, w, nchunks, nqt, nblk;
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;           // [BH][n]
    const float* beta;            // [BH][n]
    const float* gamma_q;         // [heads][d]
    const float* gamma_k;         // [heads][d]
    const float* sink;            // [heads]
    const float* gate;            // [heads]
    void* y;
    float* S_out;                 // nullable [BH][d][d]
    int32_t* cache_pos_out;       // nullable [BH][w]
    float* cache_score_out;       // nullable [BH][w]
    char* ws;
    HolaLayout L;
    // nullable: the decode memory after the call (the persistent cache at the start of the open chunk,
    // sorted by position, and the open chunk's tokens; the state itself goes to S_out)
    int32_t* st_cache_pos;        // [BH][w]
    float* st_cache_score;        // [BH][w]
    void* st_cache_k;             // [BH][w][d]
    void* st_cache_v;
    void* st_open_k;              // [BH][C][d]
    void* st_open_v;
    float* st_open_score;         // [BH][C]
};
// One decode step of the HOLA memory for every (sequence, head).
struct HolaDecodeArgs {
    int BH, heads, C, w, nopen;   // nopen = t mod C: the open chunk's tokens before this one
    int64_t t;
    const void* q;                // [BH][d]
    const void* k;
    const void* v;
    const float* alpha;           // [BH]
    const float* beta;
    const float* gamma_q;         // [heads][d]
    const float* gamma_k;
    const float* sink;            // [heads]
    const float* gate;
    void* y;                      // [BH][d]
    float* S;                     // [BH][d][d]
    int32_t* cache_pos;           // [BH][w]
    float* cache_score;
    void* cache_k;                // [BH][w][d]
    void* cache_v;
    void* open_k;                 // [BH][C][d]
    void* open_v;
    float* open_score;            // [BH][C]
};
hipError_t launch_hola_decode(const HolaDecodeArgs& a, int dtype, int d, hipStream_t stream);
struct HolaInitArgs {
    int BH, d, w;
    float* S;
    int32_t* cache_pos;
    float* cache_score;
};
hipError_t launch_hola_init(const HolaInitArgs& a, hipStream_t stream);
int device_cus();   // compute units of the current device, queried per call (256 if the query fails)
hipError_t launch_hola(const HolaArgs& a, int dtype, int d, hipStream_t stream);

struct InitArgs {
    int BH, D, d_v, lam, eta;
    float* H;
    float* s;
    int32_t* cache_pos;
    float* win_score;     // nullable
    float* cache_score;   // nullable
};

// Launchers (return hipSuccess or the launch error).  dtype: 0 = fp32, 1 = bf16.
template <typename T, int DK, int PHI>
hipError_t launch_phi_t(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_init(const InitArgs& a, hipStream_t stream);
// Query-accumulated scores of the call's keys (after the feature kernel, before the chain).
template <typename T, int DK>
hipError_t launch_qscore_t(const PrefillArgs& a, hipStream_t stream);
// The caller's second stream and events for the overlapped schedule (nullptr: sequential).
constexpr int kOverlapEvents = 9;
struct Overlap {
    hipStream_t stream;
    hipEvent_t ev[kOverlapEvents];
};
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int d, int phi_kind, hipStream_t stream,
                          hipEvent_t const* events = nullptr, const Overlap* overlap = nullptr);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, int phi_kind, hipStream_t stream);
// Chunked decode step (DecodeArgs::dec_chunk > 1), and its LDS bytes.
hipError_t launch_decode_group(const DecodeArgs& a, int dtype, int d, int phi_kind, hipStream_t stream);
size_t decode_group_lds_bytes(int d, int phi_kind, int esz, int lam, int eta, int cd);
// Register-resident decode for bf16 storage, when the cache and window fit its tiles.
bool decode_fast_fits(int d, int lam, int eta);
size_t decode_fast_lds_bytes(int d, int phi_kind);
hipError_t launch_decode_fast(const DecodeArgs& a, int d, int phi_kind, hipStream_t stream);

hipError_t launch_collide(const CollideArgs& a, int dtype, int d, hipStream_t stream);

// Read-out for bf16 storage with C = 64 or 128 (128 queries per workgroup): whether a call takes it,
// and its launcher over the chunk range [c0, c1) (c0 a multiple of 128 / C).
bool readout_fast_fits(const PrefillArgs& a, int dtype);
int readout_fast_groups_per_cu();             // workgroups of it one compute unit holds
hipError_t launch_readout_fast(const PrefillArgs& a, int d, int phi_kind, int c0, int c1, hipStream_t stream);

// LDS bytes the chain kernel uses (sized for kMaxLambda / kMaxChunk) at element size esz.
size_t chain_lds_bytes(int d, int phi_kind, int esz);
// Register-resident chain for bf16, d = 128, lambda <= 256, C <= 64 and SRE scoring (the same
// decisions and records as the general chain); LOLA_CHAIN_GENERAL in the environment turns it off.
bool chain_fast_fits(const PrefillArgs& a, int esz, int d);
hipError_t launch_chain_fast(const PrefillArgs& a, hipStream_t stream);
size_t decode_lds_bytes(int d, int phi_kind, int esz, int lam);

}  // namespace lola
