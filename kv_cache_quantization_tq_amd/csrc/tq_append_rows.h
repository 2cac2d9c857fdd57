/*
 * Which rows of one 32-token tile an append writes.  Shared by the append
 * kernel (device) and a host-side test of its arithmetic; it needs only
 * <stdint.h> and the __host__ / __device__ qualifiers (the test defines them
 * away).
 */
#ifndef TQ_APPEND_ROWS_H
#define TQ_APPEND_ROWS_H

#include <stdint.h>

/* An append of t_new tokens at row p0 of a stream of `capacity` rows, task
 * slot `slot`: the slot touches tile p0 / 32 + slot, and rows [*jlo, *jhi)
 * of that tile receive appended tokens.  Returns false (nothing to write)
 * when p0 is negative or at or past capacity, or when the tile holds no
 * appended row below capacity; on true, 32 * tile + jhi <= capacity and
 * 0 <= jlo < jhi <= 32.  The row arithmetic is in 64 bits, so no p0, t_new
 * or slot in int32 range wraps. */
__host__ __device__ inline bool tq_append_tile_rows(int32_t p0, int32_t t_new, int32_t capacity,
                                                    int32_t slot, int32_t* tile, int32_t* jlo,
                                                    int32_t* jhi) {
  *tile = *jlo = *jhi = 0;
  if (p0 < 0 || p0 >= capacity || slot < 0) return false;
  const int64_t t = (int64_t)(p0 / 32) + slot;
  const int64_t base = 32 * t;
  if (base >= capacity) return false;
  int64_t lo = (int64_t)p0 - base, hi = (int64_t)p0 + t_new - base;
  if (lo < 0) lo = 0;
  if (hi > 32) hi = 32;
  if (base + hi > capacity) hi = capacity - base;
  if (hi <= lo) return false;
  *tile = (int32_t)t;
  *jlo = (int32_t)lo;
  *jhi = (int32_t)hi;
  return true;
}

/* The end of the appended rows below capacity: min(p0 + t_new, capacity)
 * (in 64 bits, then at most capacity). */
__host__ __device__ inline int32_t tq_append_full_end(int32_t p0, int32_t t_new, int32_t capacity) {
  const int64_t fe = (int64_t)p0 + t_new;
  return fe < capacity ? (int32_t)fe : capacity;
}

/* Whether the tile `step` tiles after `tile` is, like `tile` itself, written
 * in all 32 rows, given tile's rows [jlo, jhi) and full_end from
 * tq_append_full_end: then tq_append_tile_rows for the slot `step` further
 * on gives tile + step, 0, 32. */
__host__ __device__ inline bool tq_append_next_full(int32_t tile, int32_t jlo, int32_t jhi,
                                                    int32_t full_end, int32_t step) {
  return jlo == 0 && jhi == 32 && 32 * ((int64_t)tile + step) + 32 <= full_end;
}

#endif
