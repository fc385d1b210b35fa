"""Reader for the text fixtures under tests/golden/ (whitespace-separated
tokens, '#' comments).  Every fixture states its source in its header."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name: str) -> list[list[str]]:
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out
