// Record-header validation (host only, no HIP).  Every record is checked
// before any kernel reads it: magic, expert id, offsets -- the check the WASTE
// page describes for each expert read ("Disk streaming mimarisi": magic,
// expert id and offset range are always verified so that a truncated or
// mis-joined bank never answers with wrong weights).
#include <stdint.h>
#include <string.h>

#include "moe.h"

namespace {

uint32_t rd32(const uint8_t* p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}
uint64_t rd64(const uint8_t* p) {
  uint64_t v;
  memcpy(&v, p, 8);
  return v;
}

}  // namespace

extern "C" int moe_check_record_header(const void* header, uint64_t header_bytes,
                                       const moe_config* cfg, int32_t expected_id,
                                       uint64_t record_stride) {
  if (!header || !cfg || header_bytes < 256) return MOE_EINVAL;
  const uint8_t* h = static_cast<const uint8_t*>(header);
  const bool shared = expected_id == -1;
  if (!shared && (expected_id < 0 || expected_id >= cfg->n_experts)) return MOE_EINVAL;
  const uint64_t hidden = (uint64_t)(int64_t)cfg->hidden;
  const uint64_t inter = (uint64_t)(int64_t)(shared ? cfg->shared_inter : cfg->inter);
  if (cfg->hidden <= 0 || (shared ? cfg->shared_inter : cfg->inter) <= 0) return MOE_EINVAL;
  if (rd32(h + 0) != 0x58455251u) return MOE_EBADRECORD;                 // magic
  if (rd32(h + 4) != 1u) return MOE_EBADRECORD;                          // version
  if ((int32_t)rd32(h + 8) != expected_id) return MOE_EBADRECORD;        // expert id
  if (rd32(h + 12) != hidden || rd32(h + 16) != inter) return MOE_EBADRECORD;
  if (rd32(h + 20) != 64u || rd32(h + 24) != 4u || rd32(h + 28) != 64u) return MOE_EBADRECORD;
  const uint64_t sec = (inter / 64) * (hidden / 64) * 2304ull;
  const uint64_t gate = rd64(h + 32), up = rd64(h + 40), down = rd64(h + 48), end = rd64(h + 56);
  if (gate != 256 || up != gate + sec || down != up + sec || end != down + sec)
    return MOE_EBADRECORD;
  if (end > record_stride) return MOE_EBADRECORD;
  const uint32_t crc = rd32(h + 64), hflags = rd32(h + 68);
  if (hflags > 1u || (hflags == 0u && crc != 0u)) return MOE_EBADRECORD;   // checksum field
  for (int i = 72; i < 256; ++i)
    if (h[i] != 0) return MOE_EBADRECORD;                                // reserved bytes
  return MOE_OK;
}
