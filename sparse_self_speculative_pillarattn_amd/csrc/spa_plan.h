// spa_plan.h -- work-plan records written by the host planner into the
// caller's workspace and read by the kernels.  Internal to libspa.
#pragma once
#include <stdint.h>

namespace spa {

enum : int32_t { KIND_DRAFT = 0, KIND_VERIFY = 1 };

// One request of the batch (32 bytes).
struct ReqDesc {
  int32_t L;          // tokens in context (includes the k+1 verify tokens)
  int32_t row0;       // first q / o / lse row
  int32_t kind;       // KIND_DRAFT or KIND_VERIFY
  int32_t nsplit;     // work items per KV head (1 = outputs written directly)
  int64_t part_row0;  // first split-K partial row (rows of d floats) of this request
  int64_t off;        // verify: logits element offset; draft: idx element offset
  int32_t list_len;   // draft: list entries per KV head; verify: K_r to select
  int32_t pad_;
};

// One attention work item (16 bytes): KV head g of request r over
// positions [begin, end) (verify) or list entries [begin, end) (draft).
// qi selects the single query row of an fp32 verify item (VALU path).
struct WorkItem {
  int32_t r;
  uint8_t g;
  uint8_t qi;
  uint16_t split;
  int32_t begin;
  int32_t end;
};

// One split-K merge group: request r, KV head g (8 bytes).
struct MergeItem {
  int32_t r;
  int32_t g;
};

// One verify request's selection job for one KV head (48 bytes).
struct TopkItem {
  int32_t r;
  int32_t g;
  int32_t L;
  int32_t K;
  int64_t pbar_off;    // element offset of this (r, g) row of averaged scores
  int64_t idx_off;     // element offset of the [K] output list
  int64_t logits_off;  // element offset of the request's [(k+1)][H_q][L] logits
  int32_t lse_row0;    // first lse row of the request
  int32_t pad_;
};

// One averaging block: TopkItem t, positions [j0, j0 + AVG_SPAN).
struct AvgItem {
  int32_t t;
  int32_t j0;
};

constexpr int AVG_SPAN = 1024;     // positions per averaging block
constexpr int VERIFY_TILE = 64;    // tokens per LDS tile of the MFMA verify path
constexpr int VERIFY_MAX_CHUNK = 2048;
constexpr int DRAFT_MAX_CHUNK = 2048;
constexpr int MAX_GROUP = 8;       // query heads per KV head handled by the VALU path
constexpr int MAX_ROW_TILES = 8;   // 16-row MFMA tiles (one wave each, 512 threads max)

}  // namespace spa
