// Internal declarations shared by the host and device halves of libsb.
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdint>
#include <map>
#include <string>
#include <unordered_map>
#include <vector>

#include "sb.h"

namespace sb {

int fail(int status, const char* fmt, ...);   // records sb_last_error, returns status

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

inline size_t dtype_size(int dt) { return dt == SB_BF16 ? 2 : 4; }

// Attention work decomposition (shared by the work-list builder and the kernel).
// Every work item is one workgroup of kWaves waves:
//  * MODE_ROWS: a tile of up to 64 (token, head) rows of one request and K/V
//    head against keys [0, ke); each wave owns 16 rows.
//  * MODE_RUNS: the <= 16 rows of one request and K/V head against a run of
//    keys [kb, ke): a whole number of kUnitKeys-key units (the request's last
//    unit may be short).  The waves take interleaved 32-key chunks of each
//    unit and merge their states at its end, so each unit is reduced the same
//    way wherever it falls.  A request with more than one unit leaves one
//    partial state per unit (index ITEM_PART + unit - kb / kUnitKeys), merged
//    by the combine step in unit order: results depend only on the request,
//    never on how the builder grouped units into runs.
constexpr int kRowsPerWave = 16;          // one 16x16 MFMA tile of (token, head) rows
constexpr int kWaves = 4;                 // waves per attention workgroup
constexpr int kRowsPerTile = kRowsPerWave * kWaves;       // MODE_ROWS tile (fp32)
constexpr int kRowBlocksBf16 = 2;                          // most 16-row blocks per wave in a bf16 MODE_ROWS tile
// A batch with at least this many 64-row tiles takes bf16 tiles of kRowBlocksBf16 blocks per wave (each
// staged K/V tile then serves more rows); fewer tiles keep one block per wave (more, shorter items).
constexpr int kRowBlocksMinTiles = 1024;
constexpr int kUnitKeys = 512;            // keys per independently reduced unit
constexpr int kTargetRuns = 512;          // runs per launch the builder aims at (balance vs. run length)
// An item also carries its request's first row, cached-token count and slot base (the
// request-level metadata a workgroup would otherwise fetch through two more dependent
// loads before its first q/K/V load); a group carries the request's first row.
constexpr int kItemInts = 12;
constexpr int kGroupInts = 8;
enum { ITEM_REQ = 0, ITEM_KVH, ITEM_MODE, ITEM_ROW0, ITEM_NROWS, ITEM_KB, ITEM_KE, ITEM_PART,
       ITEM_TOK0, ITEM_CTX, ITEM_SLOT0, ITEM_RB };
enum { MODE_ROWS = 0, MODE_RUNS = 1 };
enum { GRP_REQ = 0, GRP_KVH, GRP_ROW0, GRP_NROWS, GRP_PART0, GRP_NPARTS, GRP_TOK0 };

// Upper bound of the units (and so of the partials and runs) of a batch of at most B requests holding
// `keys` keys in all, per K/V head: every request adds at most one short unit.
inline int64_t max_units_bound(int64_t nkv, int64_t B, int64_t keys) { return nkv * (keys / kUnitKeys + B); }

int validate_dims(const sb_model_dims* d);

}  // namespace sb

struct sb_kv {
    struct Res {
        int64_t base;
        int64_t len;       // physical slots (max_tokens rounded up to 8)
        int32_t max_tokens;
    };
    int64_t n_slots = 0, arena_slots = 0;
    int32_t n_layers = 0, nkv = 0, d = 0, dtype = 0;
    void* k = nullptr;
    void* v = nullptr;
    hipStream_t stream = nullptr;
    int64_t n_rsrv = 0;
    int64_t n_compactions = 0;
    std::unordered_map<int64_t, Res> live;
    std::map<int64_t, int64_t> by_base;    // base slot -> request id
};
