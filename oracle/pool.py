"""Oracle of the host page pool and tag tracker (test infrastructure only:
tests/ and bench.py's baseline leg use it; the product path never does).

Plain definition, list-based: every physical page carries a 32-bit tag that
changes when the page is handed out again, and a request keeps the pages and
tags it was given (manulx.blog, "Công thức của Cloudflare để phục vụ Kimi và
GLM", section "Bảo vệ bộ nhớ đệm dùng chung"; remio.ai, section "Sicherheit
gemeinsamer KV-Caches wird zum Produktionsthema"). Reading of what the pages
leave open: one global counter stamps every hand-out (++counter, 32-bit,
wrapping); free pages form a stack, the most recently freed handed out
first; a pool without tracking stamps nothing (the no-op tracker).
"""


class OraclePagePool:
    def __init__(self, num_pages, initial_order=None, tag_start=0, track_tags=True):
        if num_pages <= 0:
            raise ValueError("num_pages must be positive")
        order = list(range(num_pages)) if initial_order is None else [int(p) for p in initial_order]
        if sorted(order) != list(range(num_pages)):
            raise ValueError("initial_order is not a permutation")
        self.num_pages = num_pages
        self.tags = [0] * num_pages
        self.in_use = [False] * num_pages
        self.free_stack = list(reversed(order))   # last element is handed out next
        self.counter = tag_start & 0xFFFFFFFF
        self.track = bool(track_tags)

    @property
    def num_free(self):
        return len(self.free_stack)

    def alloc(self, n):
        """(pages, tags) of n hand-outs; MemoryError (nothing handed out) if
        fewer than n pages are free."""
        if n < 0:
            raise ValueError("negative count")
        if n > len(self.free_stack):
            raise MemoryError("page pool exhausted")
        pages, tags = [], []
        for _ in range(n):
            p = self.free_stack.pop()
            self.in_use[p] = True
            if self.track:
                self.counter = (self.counter + 1) & 0xFFFFFFFF
                self.tags[p] = self.counter
            pages.append(p)
            tags.append(self.tags[p])
        return pages, tags

    def free(self, pages):
        """Push pages back in order; ValueError (nothing freed) if an id is
        out of range, not in use, or repeated."""
        pages = [int(p) for p in pages]
        if len(set(pages)) != len(pages):
            raise ValueError("page freed twice in one call")
        for p in pages:
            if not (0 <= p < self.num_pages) or not self.in_use[p]:
                raise ValueError(f"page {p} is not in use")
        for p in pages:
            self.in_use[p] = False
            self.free_stack.append(p)
