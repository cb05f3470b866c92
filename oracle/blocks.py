"""Plain reference model of the block manager's policy — TEST INFRASTRUCTURE.

Written from the pages' description, with lists and dicts and no attempt at
speed; the library's C++ manager (``pa_bm_*``) must make exactly the same
choices (block ids, slots, copy-on-write pairs, free counts).

Rules, as the pages state them:
 - all blocks exist from the start in one pool; each counts the requests
   using it ("大模型推理优化学习笔记", "逐出（LRU）");
 - a request's new tokens need ceil(tokens / block_size) blocks in all, the
   missing ones taken from the free queue and recorded in its table, the call
   failing if too few are free (vLLM architecture summary, "第一部分：LLM 引擎核心",
   allocate_slots: 17 new tokens -> ceil(17/16) = 2 blocks);
 - a full block is identified by the previous block's identity, its own
   tokens and a salt — so by the salt and every token from the start of the
   sequence through the block; a prompt reuses the longest run of identified
   blocks from its start; a block that is not full is never reused
   ("大模型推理优化学习笔记", "块哈希"; vLLM architecture summary, "第二部分：進階功能",
   Prefix Caching). This model compares those token runs directly (no hash);
 - a released block with no users goes to the tail of the free queue and
   keeps its identity, so it can still be reused; new blocks come from the
   head, losing their identity then ("大模型推理优化学习笔记", "逐出（LRU）");
 - a fork shares every block; a shared block that is not full is copied
   before a request appends to it ("从静态批处理到状态化推理集群", "Prefix reuse").

Readings where the pages are silent: the pool's free queue starts in block-id
order; a request's blocks are released last block first; the last prompt
token is never served from the cache (it has to be computed); among equal
full blocks the first one registered is the one reuse finds.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Tuple


class OutOfBlocks(Exception):
    pass


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16):
        self.bs = block_size
        self.ref = [0] * num_blocks
        self.tokens: List[List[int]] = [[] for _ in range(num_blocks)]
        # identity of a registered full block: (salt, all tokens from the start
        # through the block), with its registration order
        self.ident: Dict[int, Tuple] = {}
        self.order = 0
        self.free: List[int] = list(range(num_blocks))  # head = index 0
        self.reqs: Dict[int, Dict] = {}

    # ---- helpers ----
    def _alloc(self) -> int:
        b = self.free.pop(0)
        self.ident.pop(b, None)
        self.ref[b] = 1
        self.tokens[b] = []
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def _take(self, b: int) -> None:
        if self.ref[b] == 0:
            self.free.remove(b)
        self.ref[b] += 1

    def _find(self, salt: int, run) -> int:
        k = (salt, tuple(run))
        for b in sorted(self.ident, key=lambda x: self.ident[x][1]):
            if self.ident[b][0] == k:
                return b
        return -1

    # ---- operations ----
    def add_request(self, req: int, prompt: List[int], salt: int = 0) -> int:
        assert req not in self.reqs
        n = len(prompt)
        blocks: List[int] = []
        for i in range((n - 1) // self.bs if n > 0 else 0):
            b = self._find(salt, prompt[:(i + 1) * self.bs])
            if b < 0:
                break
            blocks.append(b)
        for b in blocks:
            self._take(b)
        self.reqs[req] = {"blocks": blocks, "n": len(blocks) * self.bs, "salt": salt}
        return len(blocks) * self.bs

    def append(self, req: int, toks: List[int]) -> Tuple[List[int], Optional[Tuple[int, int]]]:
        r = self.reqs[req]
        k = len(toks)
        if k == 0:
            return [], None
        total = r["n"] + k
        need = -(-total // self.bs) - len(r["blocks"])
        cow = r["n"] % self.bs != 0 and self.ref[r["blocks"][-1]] > 1
        if need + (1 if cow else 0) > len(self.free):
            raise OutOfBlocks()
        pair = None
        if cow:
            src = r["blocks"][-1]
            dst = self._alloc()
            self.tokens[dst] = list(self.tokens[src])
            self._release(src)
            r["blocks"][-1] = dst
            pair = (src, dst)
        slots = []
        for t in toks:
            pos = r["n"]
            if pos % self.bs == 0:
                r["blocks"].append(self._alloc())
            b = r["blocks"][pos // self.bs]
            slots.append(b * self.bs + pos % self.bs)
            self.tokens[b].append(t)
            r["n"] += 1
            if len(self.tokens[b]) == self.bs:
                run = [t for x in r["blocks"][:pos // self.bs + 1] for t in self.tokens[x]]
                if self._find(r["salt"], run) < 0:
                    self.order += 1
                    self.ident[b] = ((r["salt"], tuple(run)), self.order)
        return slots, pair

    def fork(self, parent: int, child: int) -> None:
        assert child not in self.reqs
        p = self.reqs[parent]
        for b in p["blocks"]:
            self._take(b)
        self.reqs[child] = {"blocks": list(p["blocks"]), "n": p["n"], "salt": p["salt"]}

    def free_request(self, req: int) -> None:
        r = self.reqs.pop(req)
        for b in reversed(r["blocks"]):
            self._release(b)

    def info(self, req: int) -> Tuple[int, List[int]]:
        r = self.reqs[req]
        return r["n"], list(r["blocks"])

    @property
    def num_free(self) -> int:
        return len(self.free)
