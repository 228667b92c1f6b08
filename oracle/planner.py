"""Oracle planners: the per-step tile plan and the static split baseline
(test infrastructure).

What the pages fix: each decode step a planner cuts the requests' KV ranges
into uniform tiles and distributes them among the thread blocks by the
current KV lengths, and the assignment is rebuilt as the lengths change
([ES-why]; [ZH-da]: a persistent kernel assigns tiles at every decode step by
the actual KV length).  The comparison point is a fixed split-KV / static
split-k schedule ([EN-vllm]; [ES-why]), which leaves units idle or launches
empty chunks for short requests.

What they leave open, and the reading taken here:
  * tile order: request-major in input order, tile j of request b covering
    tokens [j*tile_len, min((j+1)*tile_len, len_b));
  * distribution: a contiguous balanced split of that tile sequence over the
    W workgroups, the first (T mod W) workgroups taking one extra tile
    (the same cut as numpy.array_split);
  * consecutive tiles of one request inside one workgroup form one work
    item; requests covered by more than one item get partial slots numbered
    in global item order, the others write their output directly (slot -1);
  * static baseline: request b is cut into S chunks
    [floor(c*len_b/S), floor((c+1)*len_b/S)), one workgroup per chunk, W = B*S;
    empty chunks give that workgroup no item.

Plan layout (int32), shared with the C library as a data format only:
  header  [VERSION=1, B, tile_len, W, T, N, P, 0]   (tile_len 0 = static plan)
  wg_ptr  [W+1]      items of workgroup w are wg_ptr[w] .. wg_ptr[w+1]-1
  items   [N][4]     (b, kv_begin, kv_end, slot)
  req_part_ptr [B+1] partial slots of request b are req_part_ptr[b] .. [b+1]-1
"""

from dataclasses import dataclass
from typing import List, Tuple

VERSION = 1


@dataclass
class Plan:
    batch: int
    tile_len: int
    n_workgroups: int
    n_tiles: int
    items: List[Tuple[int, int, int, int]]   # (b, kv_begin, kv_end, slot)
    wg_ptr: List[int]
    req_part_ptr: List[int]

    @property
    def n_items(self):
        return len(self.items)

    @property
    def n_partials(self):
        return self.req_part_ptr[-1]

    def to_list(self):
        """The flat int32 layout described in the module docstring."""
        out = [VERSION, self.batch, self.tile_len, self.n_workgroups,
               self.n_tiles, self.n_items, self.n_partials, 0]
        out += list(self.wg_ptr)
        for it in self.items:
            out += list(it)
        out += list(self.req_part_ptr)
        return out


def _number_slots(batch, items_per_wg):
    """Flatten per-workgroup item lists and number the partial slots."""
    count = [0] * batch
    for wg in items_per_wg:
        for (b, _, _) in wg:
            count[b] += 1
    items, wg_ptr = [], [0]
    slot_of_req = [[] for _ in range(batch)]
    next_slot = 0
    for wg in items_per_wg:
        for (b, k0, k1) in wg:
            if count[b] > 1:
                slot = next_slot
                next_slot += 1
                slot_of_req[b].append(slot)
            else:
                slot = -1
            items.append((b, k0, k1, slot))
        wg_ptr.append(len(items))
    # slots are handed out in global item order; gather each request's slots
    req_part_ptr = [0]
    for b in range(batch):
        req_part_ptr.append(req_part_ptr[-1] + len(slot_of_req[b]))
    return items, wg_ptr, req_part_ptr, slot_of_req


def plan_dynamic(seq_lens, tile_len, n_workgroups):
    """Uniform tiles spread evenly over the workgroups ([ES-why]; [ZH-da])."""
    seq_lens = [int(x) for x in seq_lens]
    B, W = len(seq_lens), int(n_workgroups)
    if B < 1 or tile_len < 1 or W < 1 or any(L < 1 for L in seq_lens):
        raise ValueError("invalid plan arguments")
    # 1. the request-major tile sequence
    tiles = []
    for b, L in enumerate(seq_lens):
        n = (L + tile_len - 1) // tile_len
        for j in range(n):
            tiles.append((b, j * tile_len, min((j + 1) * tile_len, L)))
    T = len(tiles)
    # 2. contiguous balanced split: first r workgroups take q+1 tiles
    q, r = divmod(T, W)
    per_wg, pos = [], 0
    for w in range(W):
        take = q + (1 if w < r else 0)
        chunk = tiles[pos:pos + take]
        pos += take
        # 3. consecutive tiles of one request merge into one item
        merged = []
        for (b, k0, k1) in chunk:
            if merged and merged[-1][0] == b and merged[-1][2] == k0:
                merged[-1] = (b, merged[-1][1], k1)
            else:
                merged.append((b, k0, k1))
        per_wg.append(merged)
    items, wg_ptr, rpp, slots = _number_slots(B, per_wg)
    # slots of a request must be contiguous for the req_part_ptr ranges;
    # with a contiguous split the items of one request are consecutive.
    for b in range(B):
        s = slots[b]
        assert s == list(range(rpp[b], rpp[b + 1])), "non-contiguous slots"
    return Plan(B, int(tile_len), W, T, items, wg_ptr, rpp)


def plan_static(seq_lens, n_splits):
    """Fixed split per request, one workgroup per chunk ([EN-vllm]; [ES-why])."""
    seq_lens = [int(x) for x in seq_lens]
    B, S = len(seq_lens), int(n_splits)
    if B < 1 or S < 1 or any(L < 1 for L in seq_lens):
        raise ValueError("invalid plan arguments")
    per_wg = []
    for b, L in enumerate(seq_lens):
        for c in range(S):
            k0, k1 = (c * L) // S, ((c + 1) * L) // S
            per_wg.append([(b, k0, k1)] if k1 > k0 else [])
    items, wg_ptr, rpp, slots = _number_slots(B, per_wg)
    for b in range(B):
        assert slots[b] == list(range(rpp[b], rpp[b + 1]))
    n_chunks = sum(len(x) for x in per_wg)
    return Plan(B, 0, B * S, n_chunks, items, wg_ptr, rpp)
