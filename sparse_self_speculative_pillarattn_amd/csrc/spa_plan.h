// spa_plan.h -- work-plan records shared by the host planner and the kernels.
// Internal to libspa.  The plan lives in pinned host memory and the kernels
// read it in place; one record per workgroup.
#pragma once
#include <stdint.h>

namespace spa {

// ---- attention launch ------------------------------------------------------
enum : int32_t {
  KIND_NOP = 0,     // no work (the planner writes none; a workgroup that draws one moves on)
  KIND_VERIFY = 1,  // full attention of the verify rows over positions [begin, end)
  KIND_DRAFT = 2,   // sparse attention of one draft row over list entries [begin, end)
};

// One attention work item (64 bytes): KV head g of request r.
struct Item {
  int32_t kind;
  int32_t r;          // the request's page-table row
  int32_t g;
  int32_t qi;         // fp32 verify items: the single query row handled
  int32_t begin;      // positions (verify) or list entries (draft)
  int32_t end;
  int32_t L;          // context length of request r
  int32_t row0;       // first q / o / lse row of request r
  int32_t nchunk;     // split-K chunks of (r, g); 1 = outputs written directly
  int32_t split;      // chunk index of this item within (r, g)
  int32_t list_len;   // draft: entries per KV head
  int32_t ng;         // MFMA draft items: KV heads g .. g+ng-1 whose lists the item holds (1 otherwise)
  int64_t off;        // verify: logits element offset of request r; draft: list offset of (r, g)
  int64_t part_row0;  // first split-K partial row of (r, g)
};

// ---- PillarAttn post-pass launch -------------------------------------------
enum : int32_t {
  POST_NOP = 0,
  POST_MERGE = 1,  // merge the split-K partials of rows [j0, j1) of (r, g) into O and LSE
  POST_AVG = 2,    // averaged exact scores of positions [j0, j1) of verify (r, g)
};

// One post-pass item (72 bytes).  The selection launch reads the same record,
// one per verify (r, g).
struct PostItem {
  int32_t kind;
  int32_t r;
  int32_t g;
  int32_t rows_q;      // query rows of request r (k+1 verify, 1 draft)
  int32_t L;
  int32_t row0;        // first q / o / lse row of request r
  int32_t nchunk;      // split-K partials per row (1 = the LSE array is already final)
  int32_t j0, j1;      // POST_AVG: positions; POST_MERGE: rows i*G + h of (r, g)
  int32_t K;           // positions to select
  int32_t hist_slot;   // the (r, g) histogram of averaged scores, or -1 (none kept)
  int64_t part_row0;   // first split-K partial row of (r, g)
  int64_t logits_off;  // POST_AVG: logits element offset of request r
  int64_t idx_off;     // POST_AVG: element offset of the (r, g) output list
  int64_t pbar_off;    // POST_AVG: element offset of the (r, g) averaged scores
};

// ---- recallable index launch ------------------------------------------------
// One record per request (32 bytes); the launch runs one workgroup per
// (request, KV head).
struct RecallReq {
  int32_t L;          // current context length of the request
  int32_t in_count;   // stored entries per KV head
  int32_t out_count;  // output entries per KV head (members, then -1)
  int32_t pad_;
  int64_t in_off;     // element offset of the stored [H_kv][in_count] list
  int64_t out_off;    // element offset of the output [H_kv][out_count] list
};

constexpr int MAX_RECALL_LEN = 1 << 20;  // positions covered by one LDS bitmap (128 KB)

// ---- list quality launch ------------------------------------------------------
// One record per request (40 bytes); the launch runs one workgroup per
// (request, query head).
struct QualityReq {
  int32_t L;          // context length: positions [0, L) of the scored row
  int32_t n;          // list entries per KV head
  int64_t logits_off; // element offset of the request's [rows][H_q][L] logits
  int64_t list_off;   // element offset of the request's [H_kv][n] list
  int64_t p_off;      // element offset of the request's [H_q][L rounded to 4] workspace rows
  int32_t lse_row;    // LSE row of the scored row: [rows][H_q] with rows per request
  int32_t pad_;
};

// First bytes of a caller's plan buffer: the release protocol (api.cpp).  The
// device stores a call's sequence number into done[] once it no longer reads
// the records that follow the header.
struct PlanHeader {
  uint64_t magic;   // PLAN_MAGIC once a call has used the buffer
  uint64_t issued;  // sequence number of the last call that wrote the buffer
  int32_t device;   // device of that call
  int32_t drain;    // 1: that call failed after writing; drain `device` before reuse
  uint32_t need;    // done[] words that call armed (bit b: done[b])
  uint32_t pad_[9];
  uint64_t done[2]; // written by the device: [0] main release, [1] draft launch of an overlapped step
  uint64_t pad2_[22];
};
static_assert(sizeof(PlanHeader) == 256, "plan header is 256 bytes");
constexpr uint64_t PLAN_MAGIC = 0x53504150'4c414e32ull;
constexpr size_t PLAN_HEADER = sizeof(PlanHeader);
constexpr size_t WS_COUNTERS = 256;    // work counters at the start of a workspace
constexpr int AVG_SPAN = 1024;         // positions per averaging item
// Logits a step may dump and still find in the 256 MiB Infinity Cache when the
// post-pass reads them back.  Measured on the post-pass: 132 MB of logits, no
// difference between plain and streaming loads; 221 MB, plain 42.7 us against
// 55.6 us; 560 MB, plain 128 us against 95 us.
constexpr int64_t LOGITS_CACHED_BYTES = (int64_t)256 << 20;
constexpr int VERIFY_MAX_CHUNK = 2048;
constexpr int DRAFT_MAX_CHUNK = 2048;
constexpr int MAX_GROUP = 8;           // query heads per KV head on the VALU path
constexpr int TILE_TOKENS = 32;        // KV rows per LDS tile of the MFMA path
constexpr int PACK_TILES = 32;         // a packed draft item stops growing at this many tiles
constexpr int PACK_Q_BYTES = 4096;     // query rows a packed draft item stages in LDS
constexpr int MAX_ROW_TILES = 7;       // 16-row MFMA tiles (one wave each + a producer, 512 threads max)
constexpr int MAX_AVG_TERMS = 512;     // averaged (row, head) pairs per KV head
constexpr int MAX_MERGE_CHUNKS = 256;  // split-K chunks per (r, g)
constexpr int MERGE_ROWS = 8;          // rows per merge item
constexpr int SELECT_SPAN = 8192;      // scores a selection workgroup keeps in registers
constexpr int HIST_BINS = 2048;        // averaged-score histogram of a selected row: bits 30..20
constexpr int HIST_SHIFT = 20;
// Rows longer than SEL_CHUNKED_MIN scores, in a call whose attention launch
// counted their histograms, are
// selected by one workgroup per SELECT_SPAN-score chunk: a count launch (each
// chunk counts its keys above the histogram's boundary bin and stores the
// bin's keys in a region of its own), then the selection launch (the row's
// candidates gathered and ranked, each chunk's positions written at its
// offset).  A row keeps at most SEL_CAND_CAP boundary-bin keys; with more, one
// workgroup selects it alone.
constexpr int SEL_CHUNKED_MIN = 4 * SELECT_SPAN;
constexpr int SEL_CAND_CAP = 2048;
// A verify row is at most MAX_MERGE_CHUNKS * VERIFY_MAX_CHUNK positions, so a
// chunked row has at most 64 chunks: one per lane of a wave.
constexpr int SEL_MAX_ROW_CHUNKS = 64;
static_assert((int64_t)MAX_MERGE_CHUNKS * VERIFY_MAX_CHUNK <= (int64_t)SEL_MAX_ROW_CHUNKS * SELECT_SPAN,
              "every verify row fits the chunked selection");
// One chunk of a long selected row, positions [chunk * SELECT_SPAN,
// (chunk + 1) * SELECT_SPAN), with the row's fields that both launches need.
// A row's n chunks are consecutive records, chunk 0 (record `first`) first.
struct SelChunk {
  int32_t chunk;
  int32_t first;
  int32_t n;
  int32_t L;          // the row's scores
  int32_t K;          // its list length
  int32_t hist_slot;  // its histogram, boundary record and candidate counts
  int64_t pbar_off;   // its averaged scores
  int64_t idx_off;    // its list
};
static_assert(sizeof(SelChunk) == 40, "chunk record layout");
// Whether a row of L scores with a histogram is selected in chunks.
__host__ __device__ constexpr bool sel_chunked(int L) {
  return L > SEL_CHUNKED_MIN && L <= SEL_MAX_ROW_CHUNKS * SELECT_SPAN;
}

}  // namespace spa
